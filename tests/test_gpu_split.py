"""Split calls (few long rows) on the GPU against the oracle.

A window call (rlca_X_chunk or the generic scan) given a workspace, on few
long rows, cuts each row into segments: the window calls' split along T
inside one library call (the operator of the rl-triton pages' Method 1 is
associative, so the pieces join through their carry maps).  Every test runs
both forms: the chained one (one pass: each segment's workgroup publishes
its carry map and composes the published maps of the up to 64 segments
before it; up to 256 segments per row, up to 224 rows of at least 8192
steps) and the three-launch one (maps only, compose, outputs;
rlca_set_chained(False); up to 64 rows of at least 32768 steps, the call
runs unsplit otherwise), which takes over where the chained one does not
apply.  The results must match the oracle to the same tolerance as an
unsplit call, for every algorithm, with episode boundaries that fall inside
and exactly at segment borders and with carries that cross every border (no
boundaries), from 8 segments per row up to 256: the three-launch
composition then walks its 64-segment chunks one after another, and the
chained look-back its 64-segment windows.
"""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import (ALGOS, DEFAULT_PARAMS, TOL, assert_close, params32, random_inputs,
                        run_oracle, to_device)
from split_rules import chain_segments, takes_chained, torch_dtype
from test_gpu_parity import EXTREME_CASES, EXTREMES
from test_gpu_window import (affine_inputs, check_window, run_gpu_chunk, run_oracle_chunk,
                             window_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["chained", "three"], autouse=True)
def form(request):
    prev = rl.rlca_set_chained(request.param == "chained")
    yield request.param
    rl.rlca_set_chained(prev)


def workspace_for(N, T):
    ws = rl.split_workspace(N, T)
    assert ws is not None, "a call of %d x %d does not split" % (N, T)
    ws.fill_(float("nan"))
    return ws


def assert_split(ws, N, T, dtype="f32", algo="gae"):
    """The call split, in the form the thread's setting and the shape select."""
    chained = rl.rlca_set_chained(True)
    rl.rlca_set_chained(chained)
    if chained and takes_chained(N, T, dtype, algo):
        assert rl.rlca_last_launches() == 1, "the call did not take the chained form"
        assert rl.rlca_last_segments() == chain_segments(N, T, torch_dtype(dtype), algo)
        epoch = ws[:2].view(torch.int32).cpu().numpy()
        assert epoch[0] != 0 and epoch[1] == 0, "the chained call did not advance its epoch"
    else:
        S = rl.rlca_split_segments(N, T)
        if S == 1:  # more rows than the three-launch form takes: unsplit
            assert rl.rlca_last_launches() == 1 and rl.rlca_last_segments() == 1
            return
        assert rl.rlca_last_launches() == 3, "the call did not take the three-launch form"
        assert rl.rlca_last_segments() == S
        maps = ws[:2 * N * S].cpu().numpy()
        assert np.all(np.isfinite(maps)), "the call did not split"


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


def plain_by_window(algo, d, p, ws):
    """The window form with no carries: the plain call's results (returns and
    the forward mirrors with a zero bootstrap / initial value)."""
    out, _, _ = run_gpu_chunk(algo, d, p, None, with_carry_out=False, with_map=False,
                              workspace=ws)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_split_call_matches_oracle(algo, dtype):
    p = params32(dict(DEFAULT_PARAMS, gamma=0.999, lam=0.99))
    N, T = 3, 32768
    assert rl.rlca_split_segments(N, T) == 8
    for seed, p_b in ((71, 0.0), (72, 0.0005), (73, 0.01)):
        host = random_inputs(algo, N, T, seed, dtype, p_term=p_b, p_trunc=p_b, bootstrap=False)
        ref = run_oracle(algo, host, p)
        ws = workspace_for(N, T)
        print(algo, dtype, "N", N, "T", T, "boundary rate", p_b, flush=True)
        got = plain_by_window(algo, to_device(host), p, ws)
        assert_split(ws, N, T, dtype, algo)
        assert_close(got, ref, TOL[dtype], "%s/%s/split p=%g" % (algo, dtype, p_b))


@pytest.mark.parametrize("algo", ["gae", "retrace", "eligibility"])
def test_split_call_with_padded_rows(algo):
    p = params32(DEFAULT_PARAMS)
    N, T = 5, 32768
    assert rl.rlca_split_segments(N, T) == 8
    host = random_inputs(algo, N, T, 81, "f32", p_term=0.002, p_trunc=0.002, bootstrap=False)
    ref = run_oracle(algo, host, p)
    ws = workspace_for(N, T)
    got = plain_by_window(algo, padded(to_device(host), 37), p, ws)
    assert_split(ws, N, T, "f32", algo)
    assert_close(got, ref, TOL["f32"], "%s/split/padded" % algo)


def test_no_split_for_indivisible_rows_and_small_workspaces():
    p = params32(DEFAULT_PARAMS)
    # S = 1: the workspace is not touched, the call runs unsplit.
    assert rl.rlca_split_segments(3, 32767) == 1
    assert rl.rlca_split_workspace_bytes(3, 32767) == 0
    ws = torch.full((1 << 12,), float("nan"), device="cuda")
    host = random_inputs("gae", 3, 32767, 92, "f32", p_term=0.001, p_trunc=0.001)
    got = plain_by_window("gae", to_device(host), p, ws)
    assert rl.rlca_last_launches() == 1 and rl.rlca_last_segments() == 1
    assert torch.isnan(ws).all()
    assert_close(got, run_oracle("gae", host, p), TOL["f32"], "gae/odd T")
    # A call that splits, given a workspace one float short of the
    # three-launch form's (the smaller form's): refused before any launch,
    # nothing written.
    need = 12 * 3 * rl.rlca_split_segments(3, 32768)
    assert need == 12 * 3 * 8 and rl.rlca_split_workspace_bytes(3, 32768) >= need
    short = torch.full((need // 4 - 1,), float("nan"), device="cuda")
    dev = to_device(random_inputs("gae", 3, 32768, 91, "f32"))
    adv = torch.full((3, 32768), float("nan"), device="cuda")
    with pytest.raises(rl.RlcaError, match="rlca_split_workspace_bytes"):
        rl.rlca_gae_chunk(dev["rewards"], dev["values"], dev["terminated"], dev["truncated"],
                          dev["trunc_values"], gamma=p["gamma"], lam=p["lam"], advantages=adv,
                          workspace=short)
    torch.cuda.synchronize()
    assert torch.isnan(short).all() and torch.isnan(adv).all()


def test_split_and_unsplit_calls_agree():
    # The same window call with and without a workspace: equal up to rounding
    # order.
    p = params32(DEFAULT_PARAMS)
    N, T = 2, 1 << 16
    host = random_inputs("td_lambda", N, T, 93, "bf16", p_term=0.0005, p_trunc=0.0002)
    dev = to_device(host)
    c = torch.randn(N, generator=torch.Generator().manual_seed(5)).cuda()
    plain = run_gpu_chunk("td_lambda", dev, p, c)
    assert rl.rlca_split_segments(N, T) == 16
    ws = workspace_for(N, T)
    split = run_gpu_chunk("td_lambda", dev, p, c, workspace=ws)
    assert_split(ws, N, T, "bf16", "td_lambda")
    check_window(split, plain, "f32", "td_lambda/split vs unsplit")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_split_window_call_matches_oracle(algo, dtype):
    # carry in from the caller; carry out and carry map of the whole row
    p = params32(dict(DEFAULT_PARAMS, c_bar=0.95, rho_bar=1.05))
    N, T = 3, 32768
    for sparse in (False, True):
        d, c = window_inputs(algo, N, T, 501 + sparse, dtype, sparse)
        ws = workspace_for(N, T)
        print(algo, dtype, "window N", N, "T", T, "sparse", sparse, flush=True)
        got = run_gpu_chunk(algo, to_device(d), p, c.cuda(), workspace=ws)
        assert_split(ws, N, T, dtype, algo)
        check_window(got, run_oracle_chunk(algo, d, p, c), dtype,
                     "%s/%s split window sparse=%s" % (algo, dtype, sparse))


@pytest.mark.parametrize("reverse", [True, False])
def test_split_affine_scan_matches_oracle(reverse):
    N, T = 2, 65536
    assert rl.rlca_split_segments(N, T) == 16
    for p_reset, with_reset in ((0.0, False), (0.001, True)):
        al, be, rs, c = affine_inputs(N, T, 601, "f32", p_reset)
        ws = workspace_for(N, T)
        A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(), rs.cuda() if with_reset else None,
                                        reverse=reverse, carry_in=c.cuda(), workspace=ws)
        torch.cuda.synchronize()
        assert_split(ws, N, T, "f32", "affine")
        rA, rco, rcm = oracle.affine_scan(al, be, rs if with_reset else None, c,
                                          reverse=reverse)
        got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
               cm.double().cpu().numpy())
        check_window(got, ({"A": rA}, rco, rcm), "f32",
                     "affine split rev=%s p_reset=%g" % (reverse, p_reset))


# ------------------------------------------- 128 and 256 segments per row

def border_boundaries(d, algo, T, S, seed):
    """Sparse random boundaries plus boundaries at and just before several
    segment borders (the first step of a segment and the last of the one
    before), of both kinds where the algorithm takes truncations."""
    L = T // S
    g = np.random.Generator(np.random.PCG64(seed))
    term = d["terminated"].numpy().copy()
    trunc = d["truncated"].numpy().copy() if d.get("truncated") is not None else None
    for row in range(term.shape[0]):
        for k in g.choice(np.arange(1, S), size=min(12, S - 1), replace=False):
            t = int(k) * L - int(g.integers(0, 2))  # a segment's first step or the one before
            if trunc is not None and g.random() < 0.5:
                trunc[row, t] = 1
            else:
                term[row, t] = 1
    d["terminated"] = torch.from_numpy(term)
    if trunc is not None:
        d["truncated"] = torch.from_numpy(trunc)
    return d


MANY = [(2, 1 << 19, 128), (1, 1 << 20, 256)]


@pytest.mark.parametrize("N,T,S", MANY)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["gae", "retrace", "eligibility"])
def test_many_segments_match_oracle(algo, dtype, N, T, S):
    assert rl.rlca_split_segments(N, T) == S
    p = params32(dict(DEFAULT_PARAMS, gamma=0.999, lam=0.99))
    for form in ("plain", "window"):
        d, c = window_inputs(algo, N, T, 801 + S, dtype, sparse=True)
        d = border_boundaries(d, algo, T, S, 901 + S)
        ws = workspace_for(N, T)
        print(algo, dtype, "N", N, "T", T, "S", S, form, flush=True)
        if form == "plain":
            got = plain_by_window(algo, to_device(d), p, ws)
            assert_split(ws, N, T, dtype, algo)
            assert_close(got, run_oracle(algo, d, p), TOL[dtype],
                         "%s/%s S=%d plain" % (algo, dtype, S))
        else:
            got = run_gpu_chunk(algo, to_device(d), p, c.cuda(), workspace=ws)
            assert_split(ws, N, T, dtype, algo)
            check_window(got, run_oracle_chunk(algo, d, p, c), dtype,
                         "%s/%s S=%d window" % (algo, dtype, S))


ROWS = ([(algo, 100, 32768) for algo in ALGOS]
        + [(algo, 200, 32768) for algo in ("gae", "retrace", "eligibility")]
        + [(algo, 16, 16384) for algo in ("gae", "vtrace", "retrace", "eligibility")]
        + [(algo, 64, 8192) for algo in ("gae", "td_lambda", "cumsum")])


@pytest.mark.parametrize("algo,N,T", ROWS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chained_only_shapes_match_oracle(algo, dtype, N, T):
    # Shapes only the chained form splits (the three-launch form runs them
    # unsplit): 65 to 224 rows, where the launch's last workgroup waits on
    # the rows in 64-row chunks before it advances the epoch, and rows of
    # 8192 to 32767 steps.
    S = chain_segments(N, T, torch_dtype(dtype), algo)
    assert rl.rlca_split_segments(N, T) == 1 and S > 1
    p = params32(dict(DEFAULT_PARAMS, gamma=0.999, lam=0.99))
    for form in ("plain", "window"):
        d, c = window_inputs(algo, N, T, 1701 + N, dtype, sparse=True)
        d = border_boundaries(d, algo, T, S, 1801 + N)
        ws = workspace_for(N, T)
        print(algo, dtype, "N", N, "T", T, "S", S, form, flush=True)
        if form == "plain":
            got = plain_by_window(algo, to_device(d), p, ws)
            assert_split(ws, N, T, dtype, algo)
            assert_close(got, run_oracle(algo, d, p), TOL[dtype],
                         "%s/%s %dx%d plain" % (algo, dtype, N, T))
        else:
            got = run_gpu_chunk(algo, to_device(d), p, c.cuda(), workspace=ws)
            assert_split(ws, N, T, dtype, algo)
            check_window(got, run_oracle_chunk(algo, d, p, c), dtype,
                         "%s/%s %dx%d window" % (algo, dtype, N, T))


@pytest.mark.parametrize("N,chained", [(224, True), (225, False)])
def test_row_limit_of_the_chained_split(N, chained):
    # 224 rows split chained (the epoch advance waits on four 64-row
    # chunks, the last one partial); from 225 rows the call runs unsplit
    # and leaves the workspace untouched.
    T = 32768
    p = params32(DEFAULT_PARAMS)
    host = random_inputs("gae", N, T, 2001 + N, "f32", p_term=0.001, p_trunc=0.001,
                         bootstrap=False)
    assert (rl.split_workspace(N, T) is not None) == chained
    ws = workspace_for(N, T) if chained else torch.full((1 << 12,), float("nan"),
                                                        device="cuda")
    print("gae f32 N", N, "T", T, "chained", chained, flush=True)
    got = plain_by_window("gae", to_device(host), p, ws)
    if chained:
        assert_split(ws, N, T, "f32", "gae")
    else:
        assert rl.rlca_last_launches() == 1 and rl.rlca_last_segments() == 1
        assert torch.isnan(ws).all()
    assert_close(got, run_oracle("gae", host, p), TOL["f32"], "gae/%d rows" % N)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reverse", [True, False])
def test_many_rows_affine_scan(reverse, dtype):
    N, T = 100, 32768
    S = chain_segments(N, T, torch_dtype(dtype), "affine")
    assert rl.rlca_split_segments(N, T) == 1 and S > 1
    al, be, rs, c = affine_inputs(N, T, 1901, dtype, 0.0005)
    L = T // S
    rs = rs.clone()
    rs[::2, torch.as_tensor(L * np.arange(1, S))] = 1  # resets at segment borders, even rows
    ws = workspace_for(N, T)
    print("affine", dtype, "reverse", reverse, "N", N, "S", S, flush=True)
    A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(), rs.cuda(), reverse=reverse,
                                    carry_in=c.cuda(), workspace=ws)
    torch.cuda.synchronize()
    assert_split(ws, N, T, dtype, "affine")
    rA, rco, rcm = oracle.affine_scan(al, be, rs, c, reverse=reverse)
    got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
           cm.double().cpu().numpy())
    check_window(got, ({"A": rA}, rco, rcm), dtype,
                 "affine %dx%d rev=%s" % (N, T, reverse))


@pytest.mark.parametrize("N,T,S", MANY)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reverse", [True, False])
def test_many_segments_affine_scan(reverse, dtype, N, T, S):
    assert rl.rlca_split_segments(N, T) == S
    for p_reset, form in ((0.0, "window"), (0.0005, "plain"), (0.0005, "window")):
        al, be, rs, c = affine_inputs(N, T, 611 + S, dtype, p_reset)
        L = T // S
        if p_reset:  # resets at segment borders too
            rs = rs.clone()
            rs[:, torch.as_tensor(L * np.arange(3, S, 7))] = 1
            rs[:, torch.as_tensor(L * np.arange(5, S, 11) - 1)] = 1
        cin = c if form == "window" else None
        ws = workspace_for(N, T)
        print("affine", dtype, "reverse", reverse, "S", S, form, "p_reset", p_reset, flush=True)
        A, co, cm = rl.rlca_affine_scan(al.cuda(), be.cuda(), rs.cuda() if p_reset else None,
                                        reverse=reverse,
                                        carry_in=None if cin is None else cin.cuda(),
                                        workspace=ws)
        torch.cuda.synchronize()
        assert_split(ws, N, T, dtype, "affine")
        rA, rco, rcm = oracle.affine_scan(al, be, rs if p_reset else None, cin, reverse=reverse)
        got = ({"A": A.double().cpu().numpy()}, co.double().cpu().numpy(),
               cm.double().cpu().numpy())
        check_window(got, ({"A": rA}, rco, rcm), dtype,
                     "affine S=%d rev=%s %s p_reset=%g" % (S, reverse, form, p_reset))


@pytest.mark.parametrize("N,T,S3", [(4, 65536, 16), (100, 32768, 1)])
def test_split_call_in_a_hip_graph_replays_like_eager_calls(N, T, S3):
    # A split call captured once (chained: one launch that advances the
    # workspace's epoch on every replay; three launches: both passes and the
    # compose kernel; 100 rows: chained only, unsplit in the three-launch
    # setting); every replay, with eager split calls and in-place input
    # updates in between, equals the eager call bitwise.
    p = params32(DEFAULT_PARAMS)
    assert rl.rlca_split_segments(N, T) == S3
    dev = to_device(random_inputs("gae", N, T, 701, "f32", p_term=0.0005, p_trunc=0.0005))
    args = (dev["rewards"], dev["values"], dev["terminated"], dev["truncated"],
            dev["trunc_values"])
    ws = workspace_for(N, T)
    ws_eager = workspace_for(N, T)
    adv = torch.empty(N, T, device="cuda")
    tgt = torch.empty_like(adv)
    kw = dict(gamma=p["gamma"], lam=p["lam"], with_carry_out=False, with_map=False)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rl.rlca_gae_chunk(*args, advantages=adv, targets=tgt, workspace=ws, **kw)
    torch.cuda.synchronize()
    for i in range(4):
        if i == 2:
            dev["rewards"].mul_(-0.5)
        e_adv, e_tgt, _, _ = rl.rlca_gae_chunk(*args, workspace=ws_eager, **kw)
        adv.fill_(float("nan"))
        tgt.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(adv, e_adv) and torch.equal(tgt, e_tgt), "replay %d" % i
    ref = run_oracle("gae", {k: v.cpu() for k, v in dev.items()}, p)
    assert_close({"advantages": adv.double().cpu().numpy()}, {"advantages": ref["advantages"]},
                 TOL["f32"], "gae/split graph")


@pytest.mark.parametrize("algo,which", [c for c in EXTREME_CASES
                                        if c[0] in ("gae", "vtrace", "retrace", "eligibility")])
def test_split_parameter_extremes(algo, which):
    # Split calls (both forms) at the parameter extremes of the unsplit calls'
    # test: undiscounted carries cross every segment border, gamma 0 cuts
    # every map to its first step, and unclipped ratios grow the maps past 1.
    p = params32(dict(DEFAULT_PARAMS, **EXTREMES[which]))
    N, T = 3, 32768
    host = random_inputs(algo, N, T, 4100 + which, "f32", p_term=0.0005, p_trunc=0.0005,
                         bootstrap=False)
    ws = workspace_for(N, T)
    got = plain_by_window(algo, to_device(host), p, ws)
    assert_split(ws, N, T, "f32", algo)
    assert_close(got, run_oracle(algo, host, p), TOL["f32"],
                 "%s/split %s" % (algo, EXTREMES[which]))
