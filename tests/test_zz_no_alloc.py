"""rlca_gae_chunk_noalloc, the entry point for callers that cannot allocate,
against the existing entry point it varies (rlca_gae_chunk given a caller
workspace) and against the oracle.

Two calls in a row on one device, the second on a smaller input, both large
enough to split (the library's scratch array then holds the first call's
segment maps when the second begins); then a call too short to split.  Each
result must equal rlca_gae_chunk's bitwise (the same kernels run the same
three-launch split, which the no-allocation call always takes) and match the
oracle at the fp32 bar (max|err| <= 1e-4 max|ref|).
"""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import DEFAULT_PARAMS, TOL, params32, random_inputs, rel_err

pytestmark = pytest.mark.gpu


def call(fn, d, p, cin, **kw):
    N, T = d["rewards"].shape
    outs = dict(advantages=torch.full((N, T), float("nan"), device="cuda"),
                targets=torch.full((N, T), float("nan"), device="cuda"),
                carry_out=torch.full((N,), float("nan"), device="cuda"),
                carry_map=torch.full((N, 2), float("nan"), device="cuda"))
    fn(d["rewards"], d["values"], d["terminated"], d["truncated"], d["trunc_values"],
       gamma=p["gamma"], lam=p["lam"], carry_in=cin, **outs, **kw)
    torch.cuda.synchronize()
    return outs


def test_noalloc_call_equals_the_workspace_call_twice_in_a_row():
    p = params32(dict(DEFAULT_PARAMS, gamma=0.999, lam=0.97))
    shapes = [(16, 65536), (3, 32768), (5, 1000)]  # splits 16, 8, none
    assert [rl.rlca_split_segments(N, T) for N, T in shapes] == [16, 8, 1]
    for i, (N, T) in enumerate(shapes):
        host = random_inputs("gae", N, T, 1200 + i, "f32", p_term=0.0005, p_trunc=0.0005)
        d = {k: v.cuda() for k, v in host.items()}
        g = np.random.Generator(np.random.PCG64(1300 + i))
        cin = torch.from_numpy(g.standard_normal(N).astype(np.float32))
        print("noalloc call", i, "N", N, "T", T, "segments", rl.rlca_split_segments(N, T),
              flush=True)
        got = call(rl.rlca_gae_chunk_noalloc, d, p, cin.cuda())
        ws = rl.split_workspace(N, T)
        prev = rl.rlca_set_chained(False)  # the form the no-allocation call takes
        try:
            ref_gpu = call(rl.rlca_gae_chunk, d, p, cin.cuda(), workspace=ws)
        finally:
            rl.rlca_set_chained(prev)
        for k in got:
            assert torch.equal(got[k], ref_gpu[k]), "call %d: %s differs from rlca_gae_chunk" % (i, k)
        a, t, co, cm = oracle.gae(host["rewards"], host["values"], host["terminated"],
                                  host["truncated"], host["trunc_values"], gamma=p["gamma"],
                                  lam=p["lam"], carry_in=cin, chunk=True)
        for k, r in (("advantages", a), ("targets", t), ("carry_out", co)):
            e = rel_err(got[k].double().cpu().numpy(), r)
            assert e <= TOL["f32"], "call %d: %s max|err|/max|ref| = %.3g" % (i, k, e)
        gm = got["carry_map"].double().cpu().numpy()
        assert rel_err(gm[:, 0], cm[:, 0]) <= TOL["f32"]
        assert np.max(np.abs(gm[:, 1] - cm[:, 1])) <= TOL["f32"] * max(np.max(np.abs(cm[:, 1])),
                                                                       1e-3)


def test_noalloc_call_rejects_bad_arguments_before_any_launch():
    d = {k: v.cuda() for k, v in random_inputs("gae", 4, 64, 5).items()}
    adv = torch.full((4, 64), float("nan"), device="cuda")
    with pytest.raises(rl.RlcaError) as e:
        rl.rlca_gae_chunk_noalloc(d["rewards"], d["values"], d["terminated"], d["truncated"],
                                  None, gamma=0.9, lam=0.9, advantages=adv)
    assert e.value.status == rl.RLCA_EINVAL
    torch.cuda.synchronize()
    assert torch.isnan(adv).all()
