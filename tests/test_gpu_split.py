"""Split calls (few long rows) on the GPU against the oracle.

With a workspace set, a call (plain, window form or generic scan) on at most
64 rows of at least 32768 steps cuts each row into S segments and runs them as
N * S rows of the window kernels (maps only, compose, outputs): the window
calls' split along T inside one library call.  Window calls also get the
row's carry_out and carry map from the composition.
The results must match the oracle to the same tolerance as an unsplit call,
for every algorithm, with episode boundaries that fall inside and across
segment borders and with carries that cross every border (no boundaries).
"""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import (ALGOS, DEFAULT_PARAMS, TOL, assert_close, params32, random_inputs,
                        run_gpu, run_oracle, to_device)
from test_gpu_window import (affine_inputs, check_window, run_gpu_chunk, run_oracle_chunk,
                             window_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture
def workspace():
    ws = torch.empty(1 << 16, device="cuda")
    rl.rlca_set_workspace(ws)
    yield ws
    rl.rlca_set_workspace(None)


def padded(d, pad):
    """The same inputs with every row stride `pad` elements longer."""
    out = {}
    for k, v in d.items():
        if v.dim() == 2:
            buf = torch.full((v.shape[0], v.shape[1] + pad), 7, dtype=v.dtype, device=v.device)
            buf[:, :v.shape[1]] = v
            out[k] = buf[:, :v.shape[1]]
        else:
            out[k] = v
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_split_call_matches_oracle(algo, dtype, workspace):
    p = params32(dict(DEFAULT_PARAMS, gamma=0.999, lam=0.99))
    N, T = 3, 32768
    S = rl.rlca_split_segments(N, T)
    assert S == 8
    for seed, p_b in ((71, 0.0), (72, 0.0005), (73, 0.01)):
        host = random_inputs(algo, N, T, seed, dtype, p_term=p_b, p_trunc=p_b)
        ref = run_oracle(algo, host, p)
        workspace.fill_(float("nan"))
        print(algo, dtype, "N", N, "T", T, "S", S, "boundary rate", p_b, flush=True)
        got = run_gpu(algo, to_device(host), p)
        # the first pass wrote every segment's carry map
        maps = workspace[:2 * N * S].cpu().numpy()
        assert np.all(np.isfinite(maps)), "the call did not split"
        assert_close(got, ref, TOL[dtype], "%s/%s/split p=%g" % (algo, dtype, p_b))


@pytest.mark.parametrize("algo", ["gae", "retrace", "eligibility"])
def test_split_call_with_padded_rows(algo, workspace):
    p = params32(DEFAULT_PARAMS)
    N, T = 5, 32768
    S = rl.rlca_split_segments(N, T)
    assert S == 8
    host = random_inputs(algo, N, T, 81, "f32", p_term=0.002, p_trunc=0.002)
    ref = run_oracle(algo, host, p)
    workspace.fill_(float("nan"))
    got = run_gpu(algo, padded(to_device(host), 37), p)
    assert np.all(np.isfinite(workspace[:2 * N * S].cpu().numpy()))
    assert_close(got, ref, TOL["f32"], "%s/split/padded" % algo)


def test_no_split_without_room_or_divisible_length():
    p = params32(DEFAULT_PARAMS)
    ws = torch.full((3 * 3 * 8 - 1,), float("nan"), device="cuda")  # one float short
    rl.rlca_set_workspace(ws)
    try:
        assert rl.rlca_split_segments(3, 32768) == 8
        host = random_inputs("gae", 3, 32768, 91, "f32", p_term=0.001, p_trunc=0.001)
        got = run_gpu("gae", to_device(host), p)
        assert torch.isnan(ws).all(), "a workspace too small for the split was used"
        assert_close(got, run_oracle("gae", host, p), TOL["f32"], "gae/no room")
        ws2 = torch.full((1 << 12,), float("nan"), device="cuda")
        rl.rlca_set_workspace(ws2)
        assert rl.rlca_split_segments(3, 32767) == 1
        host = random_inputs("gae", 3, 32767, 92, "f32", p_term=0.001, p_trunc=0.001)
        got = run_gpu("gae", to_device(host), p)
        assert torch.isnan(ws2).all()
        assert_close(got, run_oracle("gae", host, p), TOL["f32"], "gae/odd T")
    finally:
        rl.rlca_set_workspace(None)


def test_split_and_unsplit_calls_agree():
    # The same call with and without a workspace: equal up to rounding order.
    p = params32(DEFAULT_PARAMS)
    host = random_inputs("td_lambda", 2, 1 << 16, 93, "bf16", p_term=0.0005, p_trunc=0.0002)
    dev = to_device(host)
    plain = run_gpu("td_lambda", dev, p)
    ws = torch.empty(1 << 12, device="cuda")
    rl.rlca_set_workspace(ws)
    try:
        assert rl.rlca_split_segments(2, 1 << 16) == 16
        split = run_gpu("td_lambda", dev, p)
    finally:
        rl.rlca_set_workspace(None)
    assert_close(split, plain, TOL["f32"], "td_lambda/split vs unsplit")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_split_window_call_matches_oracle(algo, dtype, workspace):
    # carry in from the caller; carry out and carry map of the whole row
    p = params32(dict(DEFAULT_PARAMS, c_bar=0.95, rho_bar=1.05))
    N, T = 3, 32768
    S = rl.rlca_split_segments(N, T)
    for sparse in (False, True):
        d, c = window_inputs(algo, N, T, 501 + sparse, dtype, sparse)
        workspace.fill_(float("nan"))
        print(algo, dtype, "window N", N, "T", T, "S", S, "sparse", sparse, flush=True)
        got = run_gpu_chunk(algo, to_device(d), p, c.cuda())
        assert np.all(np.isfinite(workspace[:2 * N * S].cpu().numpy())), "did not split"
        check_window(got, run_oracle_chunk(algo, d, p, c), dtype,
                     "%s/%s split window sparse=%s" % (algo, dtype, sparse))


@pytest.mark.parametrize("reverse", [True, False])
def test_split_affine_scan_matches_oracle(reverse, workspace):
    N, T = 2, 65536
    S = rl.rlca_split_segments(N, T)
    assert S == 16
    for p_reset, with_reset in ((0.0, False), (0.001, True)):
        al, be, rs, c = affine_inputs(N, T, 601, "f32", p_reset)
        workspace.fill_(float("nan"))
        A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(), rs.cuda() if with_reset else None,
                                        reverse=reverse, carry_in=c.cuda())
        torch.cuda.synchronize()
        assert np.all(np.isfinite(workspace[:2 * N * S].cpu().numpy())), "did not split"
        rA, rco, rcm = oracle.affine_scan(al, be, rs if with_reset else None, c,
                                          reverse=reverse)
        got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
               cm.double().cpu().numpy())
        check_window(got, ({"A": rA}, rco, rcm), "f32",
                     "affine split rev=%s p_reset=%g" % (reverse, p_reset))


def test_split_call_in_a_hip_graph_replays_like_eager_calls(workspace):
    # The three launches of a split call (both passes and the compose kernel)
    # captured once; every replay, with eager split calls and in-place input
    # updates in between, equals the eager call bitwise.
    p = params32(DEFAULT_PARAMS)
    N, T = 4, 65536
    assert rl.rlca_split_segments(N, T) == 16
    dev = to_device(random_inputs("gae", N, T, 701, "f32", p_term=0.0005, p_trunc=0.0005))
    args = (dev["rewards"], dev["values"], dev["terminated"], dev["truncated"],
            dev["trunc_values"])
    adv = torch.empty(N, T, device="cuda")
    tgt = torch.empty_like(adv)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rl.rlca_gae(*args, gamma=p["gamma"], lam=p["lam"], advantages=adv, targets=tgt)
    torch.cuda.synchronize()
    for i in range(4):
        if i == 2:
            dev["rewards"].mul_(-0.5)
        e_adv, e_tgt = rl.rlca_gae(*args, gamma=p["gamma"], lam=p["lam"])
        adv.fill_(float("nan"))
        tgt.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(adv, e_adv) and torch.equal(tgt, e_tgt), "replay %d" % i
    ref = run_oracle("gae", {k: v.cpu() for k, v in dev.items()}, p)
    assert_close({"advantages": adv.double().cpu().numpy()}, {"advantages": ref["advantages"]},
                 TOL["f32"], "gae/split graph")
