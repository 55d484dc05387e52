"""GPU parity of the window entry points (rlca_X_chunk) and of the generic
segmented affine scan (rlca_affine_scan) against the oracle's window forms.

A window takes the scan state of the neighbouring window as carry_in and
reports carry_out and the carry map (a, b), carry_out = a + b * carry_in
(rl-triton, Technical summary, Method 3 "rollout windows"; the operator of
Method 1 is associative, so a rollout can be cut along time).  Every case
compares the GPU with the fp64 oracle on the same seeded inputs at the fp32
(1e-4) or bf16-input (1e-2) bar relative to max|ref|, over every tiling
variant with ragged row lengths, and checks that cutting a rollout into
windows chained on the GPU reproduces the one-window result.
"""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import (ALGOS, DEFAULT_PARAMS, FORWARD, TOL, assert_close, params32,
                        random_inputs, rel_err, run_gpu, to_device)
from test_gpu_parity import EXTREME_CASES, EXTREMES, misaligned_flags

pytestmark = pytest.mark.gpu

MAP_TOL = {"f32": 1e-4, "bf16": 1e-2}


def run_gpu_chunk(algo, d, p, carry_in, **kw):
    """One window call on device tensors: (outputs, carry_out, carry_map) as
    float64 numpy (outputs a dict like gpu_common.run_gpu)."""
    g = lambda k: d.get(k)
    if algo == "returns":
        out, co, cm = rl.rlca_returns_chunk(g("rewards"), g("terminated"), g("truncated"),
                                            g("trunc_values"), gamma=p["gamma"],
                                            carry_in=carry_in, **kw)
        res = {"returns": out}
    elif algo == "gae":
        adv, tgt, co, cm = rl.rlca_gae_chunk(g("rewards"), g("values"), g("terminated"),
                                             g("truncated"), g("trunc_values"), gamma=p["gamma"],
                                             lam=p["lam"], carry_in=carry_in, **kw)
        res = {"advantages": adv, "targets": tgt}
    elif algo == "td_lambda":
        out, co, cm = rl.rlca_td_lambda_chunk(g("rewards"), g("values"), g("terminated"),
                                              g("truncated"), g("trunc_values"), gamma=p["gamma"],
                                              lam=p["lam"], carry_in=carry_in, **kw)
        res = {"lambda_returns": out}
    elif algo == "vtrace":
        vs, pg, co, cm = rl.rlca_vtrace_chunk(g("rewards"), g("values"), g("log_rhos"),
                                              g("terminated"), g("truncated"), g("trunc_values"),
                                              gamma=p["gamma"], lam=p["lam"], rho_bar=p["rho_bar"],
                                              c_bar=p["c_bar"], pg_rho_bar=p["pg_rho_bar"],
                                              carry_in=carry_in, **kw)
        res = {"vs": vs, "pg_advantages": pg}
    elif algo == "retrace":
        out, co, cm = rl.rlca_retrace_chunk(g("rewards"), g("q_taken"), g("exp_q_next"),
                                            g("log_rhos"), g("terminated"), g("truncated"),
                                            gamma=p["gamma"], lam=p["lam"], c_bar=p["c_bar"],
                                            carry_in=carry_in, **kw)
        res = {"q_ret": out}
    elif algo == "eligibility":
        out, co, cm = rl.rlca_eligibility_trace_chunk(g("rewards"), g("terminated"),
                                                      g("truncated"), gamma=p["gamma"],
                                                      lam=p["lam"], carry_in=carry_in, **kw)
        res = {"traces": out}
    else:
        out, co, cm = rl.rlca_episodic_cumsum_chunk(g("rewards"), g("terminated"),
                                                    g("truncated"), carry_in=carry_in, **kw)
        res = {"sums": out}
    torch.cuda.synchronize()
    np64 = lambda t: None if t is None else t.double().cpu().numpy()
    return ({k: np64(v) for k, v in res.items() if v is not None}, np64(co), np64(cm))


def run_oracle_chunk(algo, d, p, carry_in):
    g = lambda k: None if d.get(k) is None else d[k].cpu()
    c = None if carry_in is None else carry_in.cpu()
    if algo == "returns":
        G, co, cm = oracle.returns(g("rewards"), g("terminated"), g("truncated"),
                                   g("trunc_values"), c, gamma=p["gamma"], chunk=True)
        return {"returns": G}, co, cm
    if algo == "gae":
        a, t, co, cm = oracle.gae(g("rewards"), g("values"), g("terminated"), g("truncated"),
                                  g("trunc_values"), gamma=p["gamma"], lam=p["lam"],
                                  carry_in=c, chunk=True)
        return {"advantages": a, "targets": t}, co, cm
    if algo == "td_lambda":
        G, co, cm = oracle.td_lambda(g("rewards"), g("values"), g("terminated"), g("truncated"),
                                     g("trunc_values"), gamma=p["gamma"], lam=p["lam"],
                                     carry_in=c, chunk=True)
        return {"lambda_returns": G}, co, cm
    if algo == "vtrace":
        vs, pg, co, cm = oracle.vtrace(g("rewards"), g("values"), g("log_rhos"),
                                       g("terminated"), g("truncated"), g("trunc_values"),
                                       gamma=p["gamma"], lam=p["lam"], rho_bar=p["rho_bar"],
                                       c_bar=p["c_bar"], pg_rho_bar=p["pg_rho_bar"], carry_in=c,
                                       chunk=True)
        return {"vs": vs, "pg_advantages": pg}, co, cm
    if algo == "retrace":
        q, co, cm = oracle.retrace(g("rewards"), g("q_taken"), g("exp_q_next"), g("log_rhos"),
                                   g("terminated"), g("truncated"), gamma=p["gamma"],
                                   lam=p["lam"], c_bar=p["c_bar"], carry_in=c, chunk=True)
        return {"q_ret": q}, co, cm
    if algo == "eligibility":
        z, co, cm = oracle.eligibility_trace(g("rewards"), g("terminated"), g("truncated"), c,
                                             gamma=p["gamma"], lam=p["lam"], chunk=True)
        return {"traces": z}, co, cm
    S, co, cm = oracle.episodic_cumsum(g("rewards"), g("terminated"), g("truncated"), c,
                                       chunk=True)
    return {"sums": S}, co, cm


def check_window(got, ref, dtype, what):
    (go, gco, gcm), (ro, rco, rcm) = got, ref
    tol = TOL[dtype]
    assert_close(go, ro, tol, what)
    assert rel_err(gco, rco) <= tol, "%s/carry_out %.3g" % (what, rel_err(gco, rco))
    assert rel_err(gcm[:, 0], rcm[:, 0]) <= tol, "%s/map.a %.3g" % (what, rel_err(gcm[:, 0],
                                                                               rcm[:, 0]))
    # b is a product of per-step factors (at most 1 in magnitude here): compare
    # against the largest b of the batch, or absolutely when every row is cut.
    eb = np.max(np.abs(gcm[:, 1] - rcm[:, 1])) / max(np.max(np.abs(rcm[:, 1])), 1e-3)
    assert eb <= MAP_TOL[dtype], "%s/map.b %.3g" % (what, eb)


def window_inputs(algo, N, T, seed, dtype, sparse):
    p_term, p_trunc = (0.002, 0.002) if sparse else (0.05, 0.05)
    d = random_inputs(algo, N, T, seed, dtype=dtype, p_term=p_term, p_trunc=p_trunc,
                      bootstrap=False)
    g = np.random.Generator(np.random.PCG64(seed + 23))
    c = torch.from_numpy(g.standard_normal(N).astype(np.float32))
    return d, c


def variant_lengths(v, dtype, algo):
    k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                       algo)
    tile = k * lanes
    return sorted({1, 3, 6, tile - 3, tile - 2, tile, 2 * tile, 2 * tile + 5, 2 * tile + 7})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_window_parity_every_variant(algo, dtype):
    p = params32(dict(DEFAULT_PARAMS, c_bar=0.95, rho_bar=1.05))
    for v in range(rl.rlca_num_variants()):
        for T in variant_lengths(v, dtype, algo):
            for sparse in (False, True):
                N = 37 if T < 4096 else 5
                d, c = window_inputs(algo, N, T, 1000 + 7 * v + T, dtype, sparse)
                prev = rl.rlca_set_variant(v)
                try:
                    got = run_gpu_chunk(algo, to_device(d), p, c.cuda())
                finally:
                    rl.rlca_set_variant(prev)
                assert rl.rlca_last_variant() == v
                ref = run_oracle_chunk(algo, d, p, c)
                check_window(got, ref, dtype, "%s v%d T=%d sparse=%s" % (algo, v, T, sparse))
                k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16"
                                                   else torch.float32, algo)
                if T in (k * lanes, 2 * k * lanes) and not sparse:
                    # the fixed-tile instances with flag rows off 4-byte alignment
                    prev = rl.rlca_set_variant(v)
                    try:
                        got = run_gpu_chunk(algo, misaligned_flags(to_device(d)), p, c.cuda())
                    finally:
                        rl.rlca_set_variant(prev)
                    check_window(got, ref, dtype, "%s v%d T=%d misaligned flags" % (algo, v, T))


@pytest.mark.parametrize("algo", ALGOS)
def test_window_without_carry_equals_plain_call_bitwise(algo):
    # carry_in NULL: the window instance computes exactly what the plain entry
    # point computes (the carry is 0 in both).
    p = params32(DEFAULT_PARAMS)
    d = to_device(random_inputs(algo, 19, 700, 77, bootstrap=False))
    plain = run_gpu(algo, d, p)
    win, _, _ = run_gpu_chunk(algo, d, p, None, with_carry_out=False, with_map=False)
    for k in plain:
        assert np.array_equal(plain[k], win[k]), (algo, k)


def _slice(algo, d, lo, hi):
    out = {}
    for k, v in d.items():
        if v is None:
            continue
        if k == "values":
            out[k] = v[:, lo:hi + 1]
        elif v.dim() == 2:
            out[k] = v[:, lo:hi]
        else:
            out[k] = v
    return out


@pytest.mark.parametrize("algo", ALGOS)
def test_windows_chained_on_the_gpu_reproduce_one_window(algo):
    # The rollout is cut at unaligned points; windows run from the far end
    # (reverse) or the start (forward), each taking the previous carry_out as
    # carry_in, through two device vectors used in turn.
    p = params32(DEFAULT_PARAMS)
    N, T = 23, 1500
    d = random_inputs(algo, N, T, 55, p_term=0.003, p_trunc=0.003, bootstrap=False)
    dd = to_device(d)
    cuts = [0, 1, 333, 1024, 1499, 1500]
    wins = list(zip(cuts[:-1], cuts[1:]))
    if algo not in FORWARD:
        wins = wins[::-1]
    carry, spare = torch.zeros(N, device="cuda"), torch.empty(N, device="cuda")
    pieces = {}
    for lo, hi in wins:
        o, _, _ = run_gpu_chunk(algo, _slice(algo, dd, lo, hi), p, carry, carry_out=spare,
                                with_map=False)
        carry, spare = spare, carry
        pieces[lo] = o
    ref, ref_co, _ = run_oracle_chunk(algo, d, p, None)
    got = {k: np.concatenate([pieces[lo][k] for lo, _ in sorted(wins)], axis=1) for k in ref}
    assert_close(got, ref, TOL["f32"], algo + " chained")
    assert rel_err(carry.double().cpu().numpy(), ref_co) <= TOL["f32"]


@pytest.mark.parametrize("algo", ALGOS)
def test_windows_evaluated_apart_join_through_their_maps(algo):
    # T-split: every window from carry 0 reports its map; composing the maps
    # from the far end gives each window's carry; a second pass with those
    # carries reproduces the uncut window.
    p = params32(DEFAULT_PARAMS)
    N, T = 17, 2100
    d = random_inputs(algo, N, T, 66, p_term=0.001, p_trunc=0.001, bootstrap=False)
    dd = to_device(d)
    cuts = [0, 700, 1400, 2100]
    wins = list(zip(cuts[:-1], cuts[1:]))
    maps = [run_gpu_chunk(algo, _slice(algo, dd, lo, hi), p, None, carry_map=None)[2]
            for lo, hi in wins]
    order = range(len(wins)) if algo in FORWARD else range(len(wins) - 1, -1, -1)
    c = np.zeros(N)
    carries = {}
    for i in order:
        carries[i] = c
        c = maps[i][:, 0] + maps[i][:, 1] * c
    outs = [run_gpu_chunk(algo, _slice(algo, dd, lo, hi), p,
                          torch.from_numpy(carries[i].astype(np.float32)).cuda())[0]
            for i, (lo, hi) in enumerate(wins)]
    ref, ref_co, _ = run_oracle_chunk(algo, d, p, None)
    got = {k: np.concatenate([o[k] for o in outs], axis=1) for k in ref}
    assert_close(got, ref, TOL["f32"], algo + " T-split")
    assert rel_err(c, ref_co) <= TOL["f32"]


def test_window_outputs_are_optional_and_validated():
    p = params32(DEFAULT_PARAMS)
    d = to_device(random_inputs("gae", 8, 40, 88, bootstrap=False))
    c = torch.randn(8, device="cuda")
    full = run_gpu_chunk("gae", d, p, c)
    only_map = run_gpu_chunk("gae", d, p, c, with_carry_out=False)
    assert only_map[1] is None and np.array_equal(only_map[2], full[2])
    only_carry = run_gpu_chunk("gae", d, p, c, with_map=False)
    assert only_carry[2] is None and np.array_equal(only_carry[1], full[1])
    # Overlaps are rejected before launch: carry_out with carry_map, and
    # carry_out with carry_in (no in-place update).
    buf = torch.empty(24, device="cuda")
    for co, cm in ((buf[0:8], buf[4:20].view(8, 2)), (c, None)):
        with pytest.raises(rl.RlcaError) as e:
            rl.rlca_gae_chunk(d["rewards"], d["values"], gamma=0.9, lam=0.9, carry_in=c,
                              carry_out=co, carry_map=cm, with_map=cm is not None)
        assert e.value.status == rl.RLCA_EALIAS


AFFINE_DTYPES = ["f32", "bf16"]


def affine_inputs(N, T, seed, dtype, p_reset):
    g = np.random.Generator(np.random.PCG64(seed))
    al = torch.from_numpy(g.standard_normal((N, T)).astype(np.float32))
    be = torch.from_numpy(g.uniform(-1.0, 1.0, (N, T)).astype(np.float32))
    # Mostly |beta| near 1 so that carries survive long spans.
    be = torch.where(torch.from_numpy(g.random((N, T)) < 0.8), torch.sign(be) * 0.999, be)
    rs = torch.from_numpy((g.random((N, T)) < p_reset).astype(np.uint8))
    c = torch.from_numpy(g.standard_normal(N).astype(np.float32))
    if dtype == "bf16":
        al, be = al.to(torch.bfloat16), be.to(torch.bfloat16)
    return al, be, rs, c


@pytest.mark.parametrize("dtype", AFFINE_DTYPES)
@pytest.mark.parametrize("reverse", [True, False])
def test_affine_scan_parity_every_variant(reverse, dtype):
    for v in range(rl.rlca_num_variants()):
        for T in variant_lengths(v, dtype, "affine"):
            for p_reset, with_reset in ((0.0, False), (0.01, True), (0.2, True)):
                N = 29 if T < 4096 else 4
                al, be, rs, c = affine_inputs(N, T, 3000 + v * 13 + T, dtype, p_reset)
                prev = rl.rlca_set_variant(v)
                try:
                    A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(),
                                                    rs.cuda() if with_reset else None,
                                                    reverse=reverse, carry_in=c.cuda())
                    torch.cuda.synchronize()
                finally:
                    rl.rlca_set_variant(prev)
                rA, rco, rcm = oracle.affine_scan(al, be, rs if with_reset else None, c,
                                                  reverse=reverse)
                got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
                       cm.double().cpu().numpy())
                check_window(got, ({"A": rA}, rco, rcm), dtype,
                             "affine rev=%s v%d T=%d p_reset=%g" % (reverse, v, T, p_reset))
                k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16"
                                                   else torch.float32, "affine")
                if with_reset and T in (k * lanes, 2 * k * lanes):
                    # reset flags off 4-byte alignment (the fixed-tile instances)
                    buf = torch.zeros(rs.numel() + 1, dtype=rs.dtype, device="cuda")
                    rs_mis = buf[1:].view(rs.shape)
                    rs_mis.copy_(rs.cuda())
                    prev = rl.rlca_set_variant(v)
                    try:
                        A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(), rs_mis,
                                                        reverse=reverse, carry_in=c.cuda())
                        torch.cuda.synchronize()
                    finally:
                        rl.rlca_set_variant(prev)
                    got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
                           cm.double().cpu().numpy())
                    check_window(got, ({"A": rA}, rco, rcm), dtype,
                                 "affine rev=%s v%d T=%d misaligned resets" % (reverse, v, T))


def test_affine_scan_reproduces_gae_and_eligibility_calls():
    # GAE is the reverse scan of (delta_t, gamma*lam*(1-done_t)); the
    # eligibility trace is the forward scan of (x_t, gamma*lam) reset after
    # done_{t-1}.  delta is formed here in fp32 from the pages' definition.
    p = params32(DEFAULT_PARAMS)
    d = random_inputs("gae", 31, 300, 99, bootstrap=False)
    te, tr = d["terminated"].bool(), d["truncated"].bool()
    v = d["values"]
    nv = torch.where(te, torch.zeros_like(v[:, 1:]), torch.where(tr, d["trunc_values"], v[:, 1:]))
    delta = d["rewards"] + p["gamma"] * nv - v[:, :-1]
    gl = torch.full_like(delta, p["gamma"] * p["lam"])
    A, _, _ = rl.rlca_affine_scan(delta.cuda(), gl.cuda(), (te | tr).to(torch.uint8).cuda())
    adv, _ = rl.rlca_gae(*(d[k].cuda() for k in ("rewards", "values", "terminated", "truncated",
                                                 "trunc_values")), gamma=p["gamma"], lam=p["lam"])
    ref = oracle.gae(d["rewards"], v, d["terminated"], d["truncated"], d["trunc_values"],
                     gamma=p["gamma"], lam=p["lam"])[0]
    assert rel_err(A.double().cpu().numpy(), ref) <= TOL["f32"]
    assert rel_err(adv.double().cpu().numpy(), ref) <= TOL["f32"]
    prev_done = torch.zeros_like(te)
    prev_done[:, 1:] = (te | tr)[:, :-1]
    z0 = torch.randn(31)
    Z, _, _ = rl.rlca_affine_scan(d["rewards"].cuda(), gl.cuda(), prev_done.to(torch.uint8).cuda(),
                                  reverse=False, carry_in=z0.cuda())
    ref = oracle.eligibility_trace(d["rewards"], d["terminated"], d["truncated"], z0,
                                   gamma=p["gamma"], lam=p["lam"])
    assert rel_err(Z.double().cpu().numpy(), ref) <= TOL["f32"]


def test_window_calls_in_a_hip_graph_chain_like_eager_calls():
    # A captured chain of two windows (the carry passed on device between
    # them) replays like the eager chain, with eager work and
    # synchronizations between replays and inputs changed in place.
    p = params32(DEFAULT_PARAMS)
    N, T = 40, 300
    d = to_device(random_inputs("gae", N, T, 91, p_term=0.003, p_trunc=0.003, bootstrap=False))
    late, early = _slice("gae", d, 150, T), _slice("gae", d, 0, 150)
    c0 = torch.randn(N, device="cuda")
    c1 = torch.empty(N, device="cuda")
    c2 = torch.empty(N, device="cuda")
    a_late, t_late = torch.empty(N, T - 150, device="cuda"), torch.empty(N, T - 150, device="cuda")
    a_early, t_early = torch.empty(N, 150, device="cuda"), torch.empty(N, 150, device="cuda")

    def chain(outs):
        rl.rlca_gae_chunk(late["rewards"], late["values"], late["terminated"], late["truncated"],
                          late["trunc_values"], gamma=p["gamma"], lam=p["lam"], carry_in=c0,
                          advantages=outs[0], targets=outs[1], carry_out=c1, with_map=False)
        rl.rlca_gae_chunk(early["rewards"], early["values"], early["terminated"],
                          early["truncated"], early["trunc_values"], gamma=p["gamma"],
                          lam=p["lam"], carry_in=c1, advantages=outs[2], targets=outs[3],
                          carry_out=c2, with_map=False)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            chain((a_late, t_late, a_early, t_early))
    torch.cuda.synchronize()
    for i in range(4):
        if i == 2:
            d["rewards"].mul_(-0.5)
        eager = [torch.empty_like(x) for x in (a_late, t_late, a_early, t_early)]
        chain(eager)
        e_c2 = c2.clone()
        for x in (a_late, t_late, a_early, t_early, c1, c2):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((a_late, t_late, a_early, t_early), eager):
            assert torch.equal(got, want), "replay %d" % i
        assert torch.equal(c2, e_c2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo,which", EXTREME_CASES)
def test_window_parameter_extremes(algo, which, dtype):
    # The window calls (carry in; carry and carry map out) at the parameter
    # extremes of the plain calls' test, on rows with few boundaries so that
    # the carries reach far into the window.
    p = params32(dict(DEFAULT_PARAMS, **EXTREMES[which]))
    N, T = 24, 700
    d, c = window_inputs(algo, N, T, 950 + which, dtype, True)
    got = run_gpu_chunk(algo, to_device(d), p, c.cuda())
    check_window(got, run_oracle_chunk(algo, d, p, c), dtype,
                 "%s/%s window %s" % (algo, dtype, EXTREMES[which]))
