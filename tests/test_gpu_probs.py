"""GPU parity of Retrace and V-trace from policy log-probability tables
(rlca_retrace_probs, rlca_vtrace_probs) against the oracle.

The tables are [N, T(+1), A] (rl-triton, Results: the heavier Retrace workload
loads the action probabilities at every step).  Cases cover one to 65536
actions (the largest table the entry points accept, where a tile's element
index passes 2^24 and float rounding of it starts: the slice index is then
a corrected estimate), row lengths around the 256-step tile, workgroups with
rows past N,
row strides larger than a row, table rows past element 2^31 of their buffer,
both input dtypes, the full-size workload, and out-of-range actions (NaN at
that step and every earlier step of the row).
"""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import TOL, rel_err
from reverse_linear_recurrence_amd.synth import WORKLOADS, fp32_param, make_tables, make_workload

pytestmark = pytest.mark.gpu

RP = dict(gamma=fp32_param(0.97), lam=fp32_param(0.9), c_bar=fp32_param(0.95))
VP = dict(gamma=fp32_param(0.97), lam=fp32_param(0.9), rho_bar=fp32_param(1.05),
          c_bar=fp32_param(0.95), pg_rho_bar=fp32_param(1.1))


def gpu_retrace(d, **kw):
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    out = rl.rlca_retrace_probs(g("rewards"), g("q_values"), g("actions"), g("log_pi"),
                                g("log_mu"), g("terminated"), g("truncated"), g("trunc_eq"),
                                **dict(RP, **kw))
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def ref_retrace(d, **kw):
    return oracle.retrace_probs(d["rewards"], d["q_values"], d["actions"], d["log_pi"],
                                d["log_mu"], d.get("terminated"), d.get("truncated"),
                                d.get("trunc_eq"), **dict(RP, **kw))


def gpu_vtrace(d, **kw):
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    vs, pg = rl.rlca_vtrace_probs(g("rewards"), g("values"), g("actions"), g("log_pi"),
                                  g("log_mu"), g("terminated"), g("truncated"),
                                  g("trunc_values"), **dict(VP, **kw))
    torch.cuda.synchronize()
    return vs.double().cpu().numpy(), pg.double().cpu().numpy()


def ref_vtrace(d, **kw):
    return oracle.vtrace_probs(d["rewards"], d["values"], d["actions"], d["log_pi"], d["log_mu"],
                               d.get("terminated"), d.get("truncated"), d.get("trunc_values"),
                               **dict(VP, **kw))


CASES = [(1, 1, 1), (7, 33, 2), (5, 7, 3), (11, 100, 4), (4, 129, 7), (9, 255, 18),
         (4, 256, 18), (6, 257, 18), (3, 700, 5), (2, 1024, 18), (2, 1027, 18), (3, 2100, 4),
         (5, 300, 64), (2, 260, 257)]


@pytest.mark.parametrize("mu_taken", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,T,A", CASES)
def test_retrace_probs_parity(N, T, A, dtype, mu_taken):
    for p_term, p_trunc in ((0.05, 0.05), (0.0, None)):
        d = make_tables("retrace_probs", N, T, A, seed=N * 1000 + T + A, dtype=dtype,
                        p_term=p_term, p_trunc=p_trunc, mu_taken=mu_taken)
        got, ref = gpu_retrace(d), ref_retrace(d)
        assert np.all(np.isfinite(got))
        assert rel_err(got, ref) <= TOL[dtype], (N, T, A, p_trunc, rel_err(got, ref))


@pytest.mark.parametrize("mu_taken", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,T,A", CASES)
def test_vtrace_probs_parity(N, T, A, dtype, mu_taken):
    for p_term, p_trunc in ((0.05, 0.05), (0.0, None)):
        d = make_tables("vtrace_probs", N, T, A, seed=N * 1000 + T + A + 1, dtype=dtype,
                        p_term=p_term, p_trunc=p_trunc, mu_taken=mu_taken)
        got, ref = gpu_vtrace(d), ref_vtrace(d)
        for a, b in zip(got, ref):
            assert np.all(np.isfinite(a))
            assert rel_err(a, b) <= TOL[dtype], (N, T, A, p_trunc, rel_err(a, b))


# Large action sets: slices x A of one tile above 2^24 with A = 65536 (both
# tilings: 256 steps, one wavefront per row, and 1024-step tiles), and A =
# 4096 over a ragged second tile.
LARGE = [(2, 300, 65536), (2, 256, 65536), (3, 1030, 4096), (4, 200, 4096)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,T,A", LARGE)
@pytest.mark.parametrize("algo", ["retrace_probs", "vtrace_probs"])
def test_large_action_sets(algo, N, T, A, dtype):
    # Slices one tile streams: its steps (Retrace: and the slice after them).
    tile = 1024 if T > 256 else 256
    slices = min(T, tile) + (1 if algo == "retrace_probs" else 0)
    if A == 65536:
        assert slices * A >= 1 << 24
    for mu_taken in ((False, True) if A == 65536 and dtype == "f32" else (False,)):
        d = make_tables(algo, N, T, A, seed=7000 + T + A + mu_taken, dtype=dtype, p_term=0.01,
                        p_trunc=0.01, mu_taken=mu_taken)
        print(algo, dtype, "N", N, "T", T, "A", A, "mu_taken", mu_taken, flush=True)
        if algo == "retrace_probs":
            got, ref = (gpu_retrace(d),), (ref_retrace(d),)
        else:
            got, ref = gpu_vtrace(d), ref_vtrace(d)
        for a, b in zip(got, ref):
            assert np.all(np.isfinite(a))
            assert rel_err(a, b) <= TOL[dtype], (algo, N, T, A, dtype, rel_err(a, b))
        del d
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["retrace_probs_2048x1024x18", "vtrace_probs_2048x1024x18"])
def test_full_size_workloads(name):
    w = WORKLOADS[name]
    d = make_workload(w)
    kw = {k: fp32_param(v) for k, v in w.clips.items()}
    kw.update(gamma=fp32_param(w.gamma), lam=fp32_param(w.lam))
    if w.algo == "retrace_probs":
        got, ref = gpu_retrace(d, **kw), ref_retrace(d, **kw)
        assert rel_err(got, ref) <= TOL["f32"]
    else:
        for a, b in zip(gpu_vtrace(d, **kw), ref_vtrace(d, **kw)):
            assert rel_err(a, b) <= TOL["f32"]


@pytest.mark.parametrize("mu_taken", [False, True])
def test_strided_tables_and_rows(mu_taken):
    # Rows of every array further apart than one row; results unchanged.
    N, T, A = 5, 300, 7
    d = make_tables("retrace_probs", N, T, A, seed=5, p_term=0.05, p_trunc=0.05,
                    mu_taken=mu_taken)
    ref = ref_retrace(d)
    wide = {}
    for k, v in d.items():
        pad = list(v.shape)
        pad[1] += 3
        big = torch.zeros(pad, dtype=v.dtype)
        big[:, : v.shape[1]] = v
        wide[k] = big[:, : v.shape[1]]
    assert wide["q_values"].stride(0) == (T + 4) * A
    assert rel_err(gpu_retrace(wide), ref) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["retrace_probs", "vtrace_probs"])
def test_table_rows_past_element_2_to_the_31(algo, dtype):
    # Table row offsets need 64 bits: three rows 2^30 elements apart, so the
    # last table row starts at element 2^31.  The tables are strided views
    # into one large buffer, uninitialized outside the rows, each at its own
    # odd offset inside a row slot.  Short rows (one wavefront per row) and
    # long rows (one workgroup per row).
    N, LD, A = 3, 1 << 30, 18
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for T in (100, 300):
        d = make_tables(algo, N, T, A, seed=900 + T, dtype=dtype, p_term=0.01, p_trunc=0.01)
        ref = ref_retrace(d) if algo == "retrace_probs" else ref_vtrace(d)
        tables = {k: x for k, x in d.items() if x is not None and x.dim() == 3}
        offs, off = {}, 0
        for k, x in tables.items():
            offs[k] = off + 1
            off += x.shape[1] * x.shape[2] + 64
        buf = torch.empty((N - 1) * LD + off + 8, dtype=tdt, device="cuda")
        dev = {k: (None if x is None else x.cuda()) for k, x in d.items()}
        for k, x in tables.items():
            view = buf.as_strided(tuple(x.shape), (LD, x.shape[2], 1), offs[k])
            view.copy_(x.cuda())
            dev[k] = view
        print(algo, dtype, "T", T, "last table row at element", (N - 1) * LD, flush=True)
        if algo == "retrace_probs":
            got = gpu_retrace(dev)
            assert rel_err(got, ref) <= TOL[dtype], (algo, dtype, T, rel_err(got, ref))
        else:
            got = gpu_vtrace(dev)
            for a, b in zip(got, ref):
                assert rel_err(a, b) <= TOL[dtype], (algo, dtype, T, rel_err(a, b))
        del dev, buf
        torch.cuda.empty_cache()


def test_out_of_range_action_gives_nan_where_it_reaches():
    N, T, A = 3, 40, 4
    d = make_tables("retrace_probs", N, T, A, seed=6, p_term=0.0, p_trunc=None)
    d["terminated"] = torch.zeros(N, T, dtype=torch.uint8)
    d["terminated"][1, 19] = 1          # row 1: episode ends after step 19
    d["actions"][1, 30] = A              # out of range at step 30 of row 1
    got = gpu_retrace(d)
    ok = oracle.retrace_probs(d["rewards"][[0, 2]], d["q_values"][[0, 2]], d["actions"][[0, 2]],
                              d["log_pi"][[0, 2]], d["log_mu"][[0, 2]], gamma=RP["gamma"],
                              lam=RP["lam"], c_bar=RP["c_bar"])
    assert rel_err(got[[0, 2]], ok) <= TOL["f32"]          # other rows unaffected
    # The step and every earlier step of its row: the scan cuts an episode by a
    # zero factor, and 0 * NaN is NaN, so the boundary after step 19 does not
    # stop it.  Later steps are untouched.
    assert np.all(np.isnan(got[1, :31]))
    assert np.all(np.isfinite(got[1, 31:]))


def test_empty_and_validation():
    d = make_tables("retrace_probs", 2, 3, 4, seed=7, p_trunc=0.1)
    g = {k: v.cuda() for k, v in d.items()}
    with pytest.raises(rl.RlcaError) as e:
        rl.rlca_retrace_probs(g["rewards"], g["q_values"], g["actions"], g["log_pi"],
                              g["log_mu"], g["terminated"], g["truncated"], None, gamma=0.9)
    assert e.value.status == rl.RLCA_EINVAL
    z = {k: v[:0] for k, v in g.items()}
    out = rl.rlca_retrace_probs(z["rewards"], z["q_values"], z["actions"], z["log_pi"],
                                z["log_mu"], gamma=0.9)
    assert out.shape == (0, 3)


def test_policy_table_calls_in_a_hip_graph():
    # Replays agree with eager calls (Retrace up to the order of the LDS sums
    # of the expectation; V-trace bitwise), with inputs changed in place.
    d = make_tables("retrace_probs", 9, 700, 18, seed=8, p_term=0.01, p_trunc=0.01)
    v = make_tables("vtrace_probs", 9, 700, 18, seed=9, p_term=0.01, p_trunc=0.01)
    g_ = {k: x.cuda() for k, x in d.items()}
    h_ = {k: x.cuda() for k, x in v.items()}
    q_out = torch.empty(9, 700, device="cuda")
    vs_out, pg_out = torch.empty(9, 700, device="cuda"), torch.empty(9, 700, device="cuda")

    def calls(q, vs, pg):
        rl.rlca_retrace_probs(g_["rewards"], g_["q_values"], g_["actions"], g_["log_pi"],
                              g_["log_mu"], g_["terminated"], g_["truncated"], g_["trunc_eq"],
                              out=q, **RP)
        rl.rlca_vtrace_probs(h_["rewards"], h_["values"], h_["actions"], h_["log_pi"],
                             h_["log_mu"], h_["terminated"], h_["truncated"], h_["trunc_values"],
                             vs=vs, pg_advantages=pg, **VP)

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls(q_out, vs_out, pg_out)
    torch.cuda.synchronize()
    for i in range(3):
        if i == 1:
            g_["rewards"].mul_(-0.5)
            h_["rewards"].mul_(-0.5)
        e = [torch.empty(9, 700, device="cuda") for _ in range(3)]
        calls(*e)
        for x in (q_out, vs_out, pg_out):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float((q_out - e[0]).abs().max()) <= 1e-5 * float(e[0].abs().max())
        assert torch.equal(vs_out, e[1]) and torch.equal(pg_out, e[2])


def _slice_tables(d, lo, hi, algo):
    out = {}
    for k, v in d.items():
        if k in ("q_values",) or (k == "log_pi" and algo == "retrace_probs") or k == "values":
            out[k] = v[:, lo:hi + 1]
        else:
            out[k] = v[:, lo:hi]
    return out


def gpu_window(algo, d, carry, **kw):
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    c = None if carry is None else carry.cuda()
    if algo == "retrace_probs":
        q, co, cm = rl.rlca_retrace_probs_chunk(g("rewards"), g("q_values"), g("actions"),
                                                g("log_pi"), g("log_mu"), g("terminated"),
                                                g("truncated"), g("trunc_eq"), carry_in=c, **RP,
                                                **kw)
        outs = (q,)
    else:
        vs, pg, co, cm = rl.rlca_vtrace_probs_chunk(g("rewards"), g("values"), g("actions"),
                                                    g("log_pi"), g("log_mu"), g("terminated"),
                                                    g("truncated"), g("trunc_values"), carry_in=c,
                                                    **VP, **kw)
        outs = (vs, pg)
    torch.cuda.synchronize()
    return [o.double().cpu().numpy() for o in outs], co, cm


@pytest.mark.parametrize("algo", ["retrace_probs", "vtrace_probs"])
@pytest.mark.parametrize("N,T,A", [(5, 7, 3), (6, 300, 18), (3, 1500, 5)])
def test_policy_table_windows_match_the_oracle_window_forms(algo, N, T, A):
    d = make_tables(algo, N, T, A, seed=N + T + A, p_term=0.005, p_trunc=0.005,
                    mu_taken=(T % 2 == 0))
    c = torch.from_numpy(np.random.Generator(np.random.PCG64(T)).standard_normal(N)
                         .astype(np.float32))
    outs, co, cm = gpu_window(algo, d, c)
    if algo == "retrace_probs":
        q, rco, rcm = oracle.retrace_probs(d["rewards"], d["q_values"], d["actions"],
                                           d["log_pi"], d["log_mu"], d["terminated"],
                                           d["truncated"], d["trunc_eq"], carry_in=c, chunk=True,
                                           **RP)
        refs = (q,)
    else:
        vs, pg, rco, rcm = oracle.vtrace_probs(d["rewards"], d["values"], d["actions"],
                                               d["log_pi"], d["log_mu"], d["terminated"],
                                               d["truncated"], d["trunc_values"], carry_in=c,
                                               chunk=True, **VP)
        refs = (vs, pg)
    for a, b in zip(outs, refs):
        assert rel_err(a, b) <= TOL["f32"]
    assert rel_err(co.double().cpu().numpy(), rco) <= TOL["f32"]
    assert rel_err(cm[:, 0].double().cpu().numpy(), rcm[:, 0]) <= TOL["f32"]
    eb = np.max(np.abs(cm[:, 1].double().cpu().numpy() - rcm[:, 1])) / max(
        np.max(np.abs(rcm[:, 1])), 1e-3)
    assert eb <= 1e-4


@pytest.mark.parametrize("algo", ["retrace_probs", "vtrace_probs"])
def test_policy_table_windows_chain_like_one_window(algo):
    N, T, A = 7, 1300, 9
    d = make_tables(algo, N, T, A, seed=77, p_term=0.002, p_trunc=0.002)
    whole = gpu_retrace(d) if algo == "retrace_probs" else gpu_vtrace(d)
    whole = whole if isinstance(whole, tuple) else (whole,)
    cuts = [0, 200, 1100, 1300]
    carry = None
    pieces = {}
    for lo, hi in reversed(list(zip(cuts[:-1], cuts[1:]))):
        outs, co, _ = gpu_window(algo, _slice_tables(d, lo, hi, algo), carry, with_map=False)
        carry = co.cpu()
        pieces[lo] = outs
    for j, w in enumerate(whole):
        got = np.concatenate([pieces[lo][j] for lo in cuts[:-1]], axis=1)
        assert rel_err(got, w) <= TOL["f32"], (algo, j, rel_err(got, w))


# Parameter extremes: gamma 0 and 1, lambda 0 and 1, no clipping (infinite
# clips) and tight clips, on both tilings (rows of at most 256 steps, one
# wavefront each; longer rows, 1024-step tiles).
INF = float("inf")
PROB_EXTREMES = [
    dict(gamma=0.0, lam=0.9),
    dict(gamma=1.0, lam=1.0),
    dict(gamma=1.0, lam=0.0),
    dict(gamma=0.99, lam=0.95, c_bar=INF, rho_bar=INF, pg_rho_bar=INF),
    dict(gamma=0.99, lam=0.95, c_bar=0.1, rho_bar=0.5, pg_rho_bar=2.0),
]


@pytest.mark.parametrize("T", [200, 1100])
@pytest.mark.parametrize("which", range(len(PROB_EXTREMES)))
@pytest.mark.parametrize("algo", ["retrace_probs", "vtrace_probs"])
def test_parameter_extremes(algo, which, T):
    e = {k: fp32_param(v) if v != INF else v for k, v in PROB_EXTREMES[which].items()}
    d = make_tables(algo, 6, T, 9, seed=700 + which, dtype="f32", p_term=0.01, p_trunc=0.005)
    if algo == "retrace_probs":
        e.pop("rho_bar", None)
        e.pop("pg_rho_bar", None)
        got, ref = gpu_retrace(d, **e), ref_retrace(d, **e)
        assert np.all(np.isfinite(got)) and rel_err(got, ref) <= TOL["f32"], (which, T)
    else:
        for a, b in zip(gpu_vtrace(d, **e), ref_vtrace(d, **e)):
            assert np.all(np.isfinite(a)) and rel_err(a, b) <= TOL["f32"], (which, T)
