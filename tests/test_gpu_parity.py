"""GPU parity: the HIP library against the fp64 oracle, element by element, on
the same seeded inputs.  Covers the five measured workloads at full size (in
the tiling the benchmark uses), every tiling variant on ragged lengths, the
exhaustive boundary enumeration, strided and misaligned rows, rows that
start past element 2^31 of their buffer, empty inputs, parameter extremes, and
bitwise invariants (no leak across a boundary, window end, determinism, row
permutation, power-of-two scaling)."""
import itertools

import numpy as np
import pytest
import torch

import reverse_linear_recurrence_amd as rl
from reverse_linear_recurrence_amd.synth import WORKLOADS, fp32_param, make_workload
from gpu_common import (ALGOS, DEFAULT_PARAMS, FORWARD, TOL, assert_close, params32,
                        random_inputs, rel_err, run_gpu, run_oracle, to_device)

REVERSE = tuple(a for a in ALGOS if a not in FORWARD)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _auto_variant():
    rl.rlca_set_variant(-1)
    yield
    rl.rlca_set_variant(-1)


def workload_params(w):
    p = dict(DEFAULT_PARAMS)
    p.update(gamma=w.gamma, lam=w.lam)
    p.update(w.clips)
    return params32(p)


# (The policy-table workloads have their own file, test_gpu_probs.py.)
@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if not w.algo.endswith("_probs")])
def test_workload_full_size(name):
    w = WORKLOADS[name]
    print("workload", name, flush=True)
    host = make_workload(w)
    dev = to_device(host)
    p = workload_params(w)
    algos = ("vtrace", "retrace") if w.algo == "vtrace+retrace" else (w.algo,)
    for algo in algos:
        got = run_gpu(algo, dev, p)
        ref = run_oracle(algo, host, p)
        assert_close(got, ref, TOL[w.dtype], "%s/%s" % (name, algo))
        errs = {k: rel_err(got[k], ref[k]) for k in ref}
        print(name, algo, "variant", rl.rlca_last_variant(), "rel err", errs, flush=True)


def variant_lengths(v, dtype="f32", algo="gae"):
    k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                       algo)
    tile = k * lanes
    # every residue of T mod 4 (the lane holding a row's end has 1..3 steps),
    # rows shorter than one lane's span, exactly one, two and three whole
    # tiles (the one-tile and two-tile instances, and the tile loop), and
    # ragged rows of several tiles
    return sorted({1, 2, 3, 5, 6, 7, tile // 2 + 3, tile - 4, tile - 2, tile - 1, tile,
                   tile + 1, tile + 4, 2 * tile, 2 * tile + 12, 2 * tile + 14, 3 * tile})


def misaligned_flags(dev):
    """The same inputs with every flag array moved one byte off 4-byte
    alignment (the fixed-tile instances' unaligned form)."""
    out = dict(dev)
    for k in ("terminated", "truncated"):
        f = dev.get(k)
        if f is not None:
            buf = torch.zeros(f.numel() + 1, dtype=f.dtype, device=f.device)
            out[k] = buf[1:].view(f.shape)
            out[k].copy_(f)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_every_variant_ragged_lengths(algo, dtype):
    p = params32(DEFAULT_PARAMS)
    N = 37  # not a multiple of any workgroup's row count
    for v in range(rl.rlca_num_variants()):
        for T in variant_lengths(v, dtype, algo):
            seed = 1000 * v + T
            host = random_inputs(algo, N, T, seed, dtype)
            dev = to_device(host)
            rl.rlca_set_variant(v)
            print(algo, dtype, "variant", v, "T", T, flush=True)
            got = run_gpu(algo, dev, p)
            assert rl.rlca_last_variant() == v
            ref = run_oracle(algo, host, p)
            assert_close(got, ref, TOL[dtype], "%s/%s/v%d/T%d" % (algo, dtype, v, T))
            k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16"
                                               else torch.float32, algo)
            if T in (k * lanes, 2 * k * lanes):  # fixed-tile instances, unaligned flags
                got = run_gpu(algo, misaligned_flags(dev), p)
                assert_close(got, ref, TOL[dtype], "%s/%s/v%d/T%d/misaligned flags"
                             % (algo, dtype, v, T))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_flags_read_by_every_wavefront(dtype):
    """Regression: in 512-thread workgroups some wavefronts once decoded their
    flag bytes unaligned, now and then (a reset landed 3 steps late).  Unit
    rewards, one terminal flag per row placed in turn in every wavefront's
    span, initial sums present: the episodic sum is then an exact integer
    (steps since the episode began, plus the initial sum before the first
    reset), checked bit for bit over repeated calls."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    N = 8
    for v in range(3, rl.rlca_num_variants()):
        k, lanes, _ = rl.rlca_variant_info(v, tdt, "cumsum")
        tile = k * lanes
        for T in (tile, 2 * tile, 3 * tile):
            step = max(1, T // 24)
            for rep in range(2):
                fpos = [(rep * 7 + 13 * n + step * (n + 3 * rep)) % (T - 1) for n in range(N)]
                flags = np.zeros((N, T), np.uint8)
                flags[np.arange(N), fpos] = 1
                s0 = np.arange(3, 3 + N, dtype=np.float64)
                t = np.arange(T)[None, :]
                f = np.array(fpos)[:, None]
                want = np.where(t <= f, s0[:, None] + t + 1, t - f)
                rl.rlca_set_variant(v)
                got = rl.rlca_episodic_cumsum(
                    torch.ones(N, T, dtype=tdt, device="cuda"),
                    torch.from_numpy(flags).cuda(), None,
                    torch.from_numpy(s0).to(tdt).cuda())
                torch.cuda.synchronize()
                got = got.double().cpu().numpy()
                bad = np.nonzero(got != want)
                assert bad[0].size == 0, "%s v%d T%d rep %d: row %d step %d (flag at %d)" % (
                    dtype, v, T, rep, bad[0][0], bad[1][0], fpos[bad[0][0]])


def boundary_rows(T):
    pats = np.array(list(itertools.product(range(4), repeat=T)), dtype=np.int64)
    return (pats & 1).astype(np.uint8), ((pats >> 1) & 1).astype(np.uint8)


@pytest.mark.parametrize("algo", ALGOS)
def test_exhaustive_boundaries(algo):
    # Every per-step state in {none, term, trunc, both} for T = 6 (4096 rows),
    # and the same patterns placed at the end of a longer row (T = 70), in
    # every variant.
    p = params32(DEFAULT_PARAMS)
    for T, pad in ((6, 0), (70, 64)):
        te, tr = boundary_rows(6)
        N = te.shape[0]
        host = random_inputs(algo, N, T, 77 + T, "f32", p_term=0.0, p_trunc=0.0)
        term = np.zeros((N, T), np.uint8)
        trunc = np.zeros((N, T), np.uint8)
        term[:, pad:] = te
        trunc[:, pad:] = tr
        host["terminated"] = torch.from_numpy(term)
        host["truncated"] = torch.from_numpy(trunc)
        if algo != "retrace":
            g = np.random.Generator(np.random.PCG64(5))
            host["trunc_values"] = torch.from_numpy(g.standard_normal((N, T)).astype(np.float32))
        dev = to_device(host)
        ref = run_oracle(algo, host, p)
        for v in range(rl.rlca_num_variants()):
            rl.rlca_set_variant(v)
            print(algo, "T", T, "variant", v, flush=True)
            assert_close(run_gpu(algo, dev, p), ref, TOL["f32"], "%s/T%d/v%d" % (algo, T, v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_strided_and_misaligned_rows(algo, dtype):
    # Row strides larger than T, odd row strides and odd element offsets: the
    # flag rows land at every byte alignment, bf16 rows at both half-dword
    # positions, fp32 rows at every 4-byte position inside a 16-byte line.
    p = params32(DEFAULT_PARAMS)
    for T, extra, off in ((128, 3, 1), (257, 1, 3), (64, 5, 2), (1031, 2, 1)):
        N = 29
        host = random_inputs(algo, N, T, 4242 + T, dtype)
        ref = run_oracle(algo, host, p)
        # Each 2-D input is a view into a larger device buffer: row stride
        # W + extra, first element `off` elements past the allocation start.
        strided = {k: x.cuda() for k, x in host.items() if x.dim() == 1}
        for k, x in host.items():
            if x.dim() == 2:
                buf = torch.full((off + N * (x.shape[1] + extra) + 8,), 7, dtype=x.dtype,
                                 device="cuda")
                view = buf[off:off + N * (x.shape[1] + extra)].view(N, x.shape[1] + extra)
                view = view[:, :x.shape[1]]
                view.copy_(x.cuda())
                strided[k] = view
        for v in (None, 1, 2, 3, 4):
            rl.rlca_set_variant(-1 if v is None else v)
            print(algo, dtype, "T", T, "variant", v, flush=True)
            got = run_gpu(algo, strided, p)
            assert_close(got, ref, TOL[dtype], "%s/%s/T%d/v%s" % (algo, dtype, T, v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["gae", "vtrace"])
def test_rows_past_element_2_to_the_31(algo, dtype):
    # Row offsets need 64 bits: four rows 2^30 elements apart, so the last row
    # starts at element 3 * 2^30.  Every 2-D input is a strided view into one
    # of two large buffers (floats, flags) left uninitialized outside the
    # rows; inputs sit at different offsets inside each row slot.  One tile
    # per row (T = 128) and a ragged multi-tile row (T = 4100).
    p = params32(DEFAULT_PARAMS)
    N, LD = 4, 1 << 30
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for T in (128, 4100):
        host = random_inputs(algo, N, T, 31 + T, dtype, p_term=0.01, p_trunc=0.01)
        ref = run_oracle(algo, host, p)
        two_d = {k: x for k, x in host.items() if x.dim() == 2}
        offs, off_f, off_b = {}, 0, 0
        for k, x in two_d.items():
            if x.dtype == torch.uint8:
                offs[k] = off_b + 1  # odd byte offsets: flag rows at every alignment
                off_b += x.shape[1] + 64
            else:
                offs[k] = off_f + 1  # odd element offsets
                off_f += x.shape[1] + 64
        fbuf = torch.empty((N - 1) * LD + off_f + 8, dtype=tdt, device="cuda")
        bbuf = torch.empty((N - 1) * LD + off_b + 8, dtype=torch.uint8, device="cuda")
        dev = {}
        for k, x in two_d.items():
            buf = bbuf if x.dtype == torch.uint8 else fbuf
            view = buf.as_strided((N, x.shape[1]), (LD, 1), offs[k])
            view.copy_(x.cuda())
            dev[k] = view
        print(algo, dtype, "T", T, "last row at element", (N - 1) * LD, flush=True)
        got = run_gpu(algo, dev, p)
        del dev, fbuf, bbuf
        torch.cuda.empty_cache()
        assert_close(got, ref, TOL[dtype], "%s/%s/T%d" % (algo, dtype, T))


def test_empty_and_nullable():
    r = torch.zeros(0, 16, device="cuda")
    v = torch.zeros(0, 17, device="cuda")
    adv, tgt = rl.rlca_gae(r, v, gamma=0.9, lam=0.9)
    assert adv.shape == (0, 16) and tgt.shape == (0, 16)
    for N, T in ((5, 0), (0, 0)):  # rows without steps: refused, nothing launched
        r = torch.zeros(N, T, device="cuda")
        v = torch.zeros(N, T + 1, device="cuda")
        with pytest.raises(rl.RlcaError, match="T = 0 must be >= 1") as e:
            rl.rlca_gae(r, v, gamma=0.9, lam=0.9)
        assert e.value.status == rl.RLCA_EINVAL
    host = random_inputs("gae", 9, 40, 3)
    dev = to_device(host)
    p = params32(DEFAULT_PARAMS)
    adv, tgt = rl.rlca_gae(dev["rewards"], dev["values"], dev["terminated"], dev["truncated"],
                           dev["trunc_values"], gamma=p["gamma"], lam=p["lam"],
                           with_targets=False)
    assert tgt is None
    ref = run_oracle("gae", host, p)
    assert rel_err(adv.double().cpu().numpy(), ref["advantages"]) <= TOL["f32"]
    # No flags at all.
    adv2, _ = rl.rlca_gae(dev["rewards"], dev["values"], gamma=p["gamma"], lam=p["lam"])
    ref2 = run_oracle("gae", {"rewards": host["rewards"], "values": host["values"]}, p)
    assert rel_err(adv2.double().cpu().numpy(), ref2["advantages"]) <= TOL["f32"]
    hv = random_inputs("vtrace", 9, 40, 4)
    dv = to_device(hv)
    vs, pg = rl.rlca_vtrace(dv["rewards"], dv["values"], dv["log_rhos"], dv["terminated"],
                            dv["truncated"], dv["trunc_values"], gamma=p["gamma"], lam=p["lam"],
                            with_pg=False)
    assert pg is None
    assert rel_err(vs.double().cpu().numpy(), run_oracle("vtrace", hv, p)["vs"]) <= TOL["f32"]


def test_runs_on_a_side_stream():
    host = random_inputs("td_lambda", 300, 200, 8)
    dev = to_device(host)
    p = params32(DEFAULT_PARAMS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = rl.rlca_td_lambda(dev["rewards"], dev["values"], dev["terminated"],
                                dev["truncated"], dev["trunc_values"], gamma=p["gamma"],
                                lam=p["lam"])
    s.synchronize()
    ref = run_oracle("td_lambda", host, p)
    assert rel_err(out.double().cpu().numpy(), ref["lambda_returns"]) <= TOL["f32"]


# ------------------------------------------------------------ bitwise invariants

def _perturb_after(host, algo, s, kind, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    h = {k: v.clone() for k, v in host.items()}
    N, T = h["rewards"].shape
    for k in ("rewards", "q_taken", "exp_q_next", "log_rhos", "trunc_values"):
        if k in h:
            x = h[k].float()
            x[:, s + 1:] = torch.from_numpy(g.standard_normal((N, T - s - 1)).astype(np.float32)) * 3
            h[k] = x.to(h[k].dtype)
    if "values" in h:
        x = h["values"].float()
        x[:, s + 1:] = torch.from_numpy(g.standard_normal((N, T - s)).astype(np.float32)) * 3
        h["values"] = x.to(h["values"].dtype)
    if "bootstrap" in h:
        h["bootstrap"] = h["bootstrap"] + 5
    if kind == "term" and "trunc_values" in h:
        x = h["trunc_values"].float()
        x[:, s] += 3
        h["trunc_values"] = x.to(h["trunc_values"].dtype)
    return h


@pytest.mark.parametrize("algo", REVERSE)
@pytest.mark.parametrize("kind", ["term", "trunc"])
def test_no_leak_across_boundary_bitwise(algo, kind):
    # Method 3 of the rl-triton explainer: no signal crosses an episode
    # boundary.  With a boundary at step s in every row, outputs at t <= s
    # must be bitwise identical whatever follows.
    p = params32(DEFAULT_PARAMS)
    for T, s in ((128, 40), (1024, 700), (300, 299)):
        host = random_inputs(algo, 64, T, 91, "f32", p_term=0.0, p_trunc=0.0)
        host["terminated"] = torch.zeros(64, T, dtype=torch.uint8)
        host["truncated"] = torch.zeros(64, T, dtype=torch.uint8)
        if "trunc_values" not in host and algo != "retrace":
            host["trunc_values"] = torch.randn(64, T)
        host["terminated" if kind == "term" else "truncated"][:, s] = 1
        pert = _perturb_after(host, algo, s, kind, 92)
        for v in range(rl.rlca_num_variants()):
            rl.rlca_set_variant(v)
            a = run_gpu(algo, to_device(host), p)
            b = run_gpu(algo, to_device(pert), p)
            for k in a:
                assert np.array_equal(a[k][:, :s + 1], b[k][:, :s + 1]), (algo, kind, T, v, k)


@pytest.mark.parametrize("algo", ALGOS)
def test_determinism_permutation_and_scaling_bitwise(algo):
    p = params32(dict(DEFAULT_PARAMS, gamma=0.95, lam=0.9))
    host = random_inputs(algo, 200, 256, 123, "f32")
    dev = to_device(host)
    a = run_gpu(algo, dev, p)
    b = run_gpu(algo, dev, p)
    for k in a:
        assert np.array_equal(a[k], b[k]), ("determinism", k)
    perm = torch.from_numpy(np.random.Generator(np.random.PCG64(1)).permutation(200))
    hp = {k: v[perm] for k, v in host.items()}
    c = run_gpu(algo, to_device(hp), p)
    for k in a:
        assert np.array_equal(a[k][perm.numpy()], c[k]), ("permutation", k)
    hs = {k: (v * 2 if k in ("rewards", "values", "q_taken", "exp_q_next", "trunc_values",
                             "bootstrap") else v) for k, v in host.items()}
    d = run_gpu(algo, to_device(hs), p)
    for k in a:
        assert np.array_equal(2 * a[k], d[k]), ("scaling", k)


def test_window_end_bootstrap_counted_once_bitwise():
    # With no boundary the bootstrap V_T enters A_{T-1} once; with a boundary
    # at T-1 it has no effect at all.
    p = params32(DEFAULT_PARAMS)
    for algo in ("gae", "td_lambda", "vtrace"):
        host = random_inputs(algo, 50, 130, 5, "f32", p_term=0.0, p_trunc=0.0)
        host["terminated"] = torch.zeros(50, 130, dtype=torch.uint8)
        host["terminated"][:, -1] = 1
        h2 = {k: v.clone() for k, v in host.items()}
        h2["values"][:, -1] += 9.0
        a = run_gpu(algo, to_device(host), p)
        b = run_gpu(algo, to_device(h2), p)
        for k in a:
            assert np.array_equal(a[k], b[k]), (algo, k)
    host = random_inputs("gae", 50, 130, 6, "f32", p_term=0.0, p_trunc=0.0)
    host["terminated"] = torch.zeros(50, 130, dtype=torch.uint8)
    got = run_gpu("gae", to_device(host), p)
    r, v = host["rewards"].double().numpy(), host["values"].double().numpy()
    expect = r[:, -1] + p["gamma"] * v[:, -1] - v[:, -2]
    assert np.max(np.abs(got["advantages"][:, -1] - expect)) <= 1e-5 * np.max(np.abs(expect))


@pytest.mark.parametrize("algo", ["returns", "gae", "td_lambda", "vtrace"])
def test_sparse_truncation_bootstraps_large_batch(algo):
    # Above 1M env-steps the kernels read trunc_values only at truncated
    # steps (below, as whole vectors).  Dense truncations, fp32, every
    # long-row tiling, against the oracle; the unused entries hold NaN.
    p = params32(DEFAULT_PARAMS)
    N, T = 1100, 1024
    host = random_inputs(algo, N, T, 606, "f32", p_term=0.01, p_trunc=0.02)
    tv = host["trunc_values"].clone()
    keep = (host["truncated"] != 0) & (host["terminated"] == 0)
    tv[~keep] = float("nan")
    host["trunc_values"] = tv
    ref = run_oracle(algo, host, p)
    dev = to_device(host)
    for v in (None, 2, 3, 4):
        rl.rlca_set_variant(-1 if v is None else v)
        print(algo, "variant", v, flush=True)
        assert_close(run_gpu(algo, dev, p), ref, TOL["f32"], "%s/v%s" % (algo, v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_many_workgroups_and_a_partial_last_one(algo, dtype):
    # 20003 rows of exactly one tile, in each short-row tiling: thousands of
    # workgroups (several rounds of the chip), the last with rows past N.
    p = params32(DEFAULT_PARAMS)
    N = 20003
    for v in (0, 1, 2):
        k, lanes, _ = rl.rlca_variant_info(v, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                           algo)
        T = k * lanes
        host = random_inputs(algo, N, T, 7000 + v, dtype, p_term=0.01, p_trunc=0.01)
        ref = run_oracle(algo, host, p)
        rl.rlca_set_variant(v)
        print(algo, dtype, "variant", v, "T", T, flush=True)
        assert_close(run_gpu(algo, to_device(host), p), ref, TOL[dtype],
                     "%s/%s/v%d" % (algo, dtype, v))


@pytest.mark.parametrize("algo", ALGOS)
def test_wide_variants_on_fp32_are_their_narrow_twins(algo):
    # Variants 6-8 take 8 steps per lane on bf16 only; on fp32 inputs (and for
    # V-trace on bf16) they run the kernels of variants 3-5, so the outputs
    # are equal bitwise.
    p = params32(DEFAULT_PARAMS)
    cases = [("f32", algo)] + ([("bf16", algo)] if algo == "vtrace" else [])
    for dtype, a in cases:
        host = random_inputs(a, 9, 5000, 4242, dtype)
        dev = to_device(host)
        for v in (3, 4, 5):
            assert rl.rlca_variant_info(v + 3, torch.bfloat16 if dtype == "bf16"
                                        else torch.float32, a)[0] == 4
            rl.rlca_set_variant(v)
            try:
                narrow = run_gpu(a, dev, p)
                rl.rlca_set_variant(v + 3)
                wide = run_gpu(a, dev, p)
            finally:
                rl.rlca_set_variant(-1)
            for k in narrow:
                assert np.array_equal(narrow[k], wide[k]), "%s/%s/v%d/%s" % (a, dtype, v, k)


def test_default_tiling_choice():
    # The default variant for a few shapes: one-wavefront tiles for short
    # rows, whole wavefronts per row for long ones, and on bf16 the wide twin
    # (8 steps per lane) only when the row holds one wide tile; never for
    # fp32 or V-trace.  (The choice depends on the shape, not on the data.)
    p = params32(DEFAULT_PARAMS)
    cases = [("gae", "f32", 4096, 128, 1), ("gae", "f32", 16384, 256, 2),
             ("gae", "f32", 256, 16384, 5), ("gae", "bf16", 256, 16384, 8),
             ("gae", "bf16", 512, 8192, 7), ("gae", "bf16", 1024, 2048, 6),
             ("gae", "bf16", 2048, 1024, 3), ("vtrace", "bf16", 256, 16384, 5),
             ("retrace", "bf16", 1024, 2048, 6), ("td_lambda", "f32", 2048, 1024, 3)]
    assert rl.rlca_set_variant(-1) == -1
    for algo, dtype, N, T, want in cases:
        dev = to_device(random_inputs(algo, N, T, 11, dtype))
        run_gpu(algo, dev, p)
        assert rl.rlca_last_variant() == want, (algo, dtype, N, T, rl.rlca_last_variant())


def test_hip_graph_replay_matches_eager():
    # The benchmark replays captured launches; every replay, with eager work
    # and synchronizations in between, must equal the eager call bitwise, and
    # must see inputs updated in place.
    host = random_inputs("gae", 300, 200, 9)
    dev = to_device(host)
    p = params32(DEFAULT_PARAMS)
    args = (dev["rewards"], dev["values"], dev["terminated"], dev["truncated"],
            dev["trunc_values"])
    adv = torch.empty(300, 200, device="cuda")
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
            dev["rewards"].mul_(-0.5)  # in-place input update between replays
        e_adv, e_tgt = rl.rlca_gae(*args, gamma=p["gamma"], lam=p["lam"])
        adv.fill_(float("nan"))
        tgt.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(adv, e_adv) and torch.equal(tgt, e_tgt), "replay %d" % i
    ref = run_oracle("gae", {k: v.cpu() for k, v in dev.items()}, p)
    assert rel_err(adv.double().cpu().numpy(), ref["advantages"]) <= TOL["f32"]


def test_concurrent_calls_on_two_streams():
    hosts = [random_inputs(a, 700, 300, 31 + i) for i, a in enumerate(("gae", "vtrace"))]
    devs = [to_device(h) for h in hosts]
    p = params32(DEFAULT_PARAMS)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = rl.rlca_gae(devs[0]["rewards"], devs[0]["values"], devs[0]["terminated"],
                            devs[0]["truncated"], devs[0]["trunc_values"], gamma=p["gamma"],
                            lam=p["lam"])
        with torch.cuda.stream(s2):
            b = rl.rlca_vtrace(devs[1]["rewards"], devs[1]["values"], devs[1]["log_rhos"],
                               devs[1]["terminated"], devs[1]["truncated"],
                               devs[1]["trunc_values"], gamma=p["gamma"], lam=p["lam"])
        outs.append((a, b))
    torch.cuda.synchronize()
    ra = run_oracle("gae", hosts[0], p)
    rb = run_oracle("vtrace", hosts[1], p)
    for a, b in outs:
        assert rel_err(a[0].double().cpu().numpy(), ra["advantages"]) <= TOL["f32"]
        assert rel_err(b[0].double().cpu().numpy(), rb["vs"]) <= TOL["f32"]
        assert rel_err(b[1].double().cpu().numpy(), rb["pg_advantages"]) <= TOL["f32"]


@pytest.mark.parametrize("algo", FORWARD)
@pytest.mark.parametrize("kind", ["term", "trunc"])
def test_forward_no_leak_across_boundary_bitwise(algo, kind):
    # Forward mirror of the no-leak invariant: with a boundary after step s,
    # outputs at t > s are bitwise independent of every input at t <= s and
    # of the carry-in.
    p = params32(DEFAULT_PARAMS)
    for T, s in ((128, 40), (1024, 700), (300, 0)):
        host = random_inputs(algo, 64, T, 93, "f32", p_term=0.0, p_trunc=0.0)
        host["terminated"] = torch.zeros(64, T, dtype=torch.uint8)
        host["truncated"] = torch.zeros(64, T, dtype=torch.uint8)
        host["terminated" if kind == "term" else "truncated"][:, s] = 1
        pert = {k: v.clone() for k, v in host.items()}
        pert["rewards"][:, : s + 1] += torch.randn(64, s + 1) * 3
        pert["bootstrap"] = pert["bootstrap"] + 4
        for v in range(rl.rlca_num_variants()):
            rl.rlca_set_variant(v)
            a = run_gpu(algo, to_device(host), p)
            b = run_gpu(algo, to_device(pert), p)
            for k in a:
                assert np.array_equal(a[k][:, s + 1:], b[k][:, s + 1:]), (algo, kind, T, v, k)


# Parameter extremes: no discount propagation (gamma 0), undiscounted sums
# (gamma = lambda = 1), one-step TD (lambda 0), no clipping (infinite clips) and
# tight clips with a policy-gradient clip above the others.  Every algorithm
# uses the parameters it takes; the episodic sum takes none.
INF = float("inf")
EXTREMES = [
    dict(gamma=0.0, lam=0.9),
    dict(gamma=1.0, lam=1.0),
    dict(gamma=1.0, lam=0.0),
    dict(gamma=0.5, lam=1.0),
    dict(gamma=0.99, lam=0.95, rho_bar=INF, c_bar=INF, pg_rho_bar=INF),
    dict(gamma=0.99, lam=0.95, rho_bar=0.5, c_bar=0.1, pg_rho_bar=2.0),
]


EXTREME_CASES = [(algo, i) for algo in ALGOS for i in range(len(EXTREMES))
                 if (algo != "cumsum" or i == 0) and (algo in ("vtrace", "retrace") or i < 4)]


@pytest.mark.parametrize("T", [300, 2100])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo,which", EXTREME_CASES)
def test_parameter_extremes(algo, which, dtype, T):
    p = params32(dict(DEFAULT_PARAMS, **EXTREMES[which]))
    N = 24
    host = random_inputs(algo, N, T, 900 + which, dtype, p_term=0.01, p_trunc=0.005)
    got = run_gpu(algo, to_device(host), p)
    assert_close(got, run_oracle(algo, host, p), TOL[dtype],
                 "%s/%s T=%d %s" % (algo, dtype, T, EXTREMES[which]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_non_finite_inputs(algo, dtype):
    # NaN and infinite rewards: the scan evaluates each step as alpha + beta *
    # A with beta = 0 at an episode boundary, and 0 * NaN is NaN, so a
    # non-finite value reaches every step on the far side of it in scan order,
    # across boundaries too, where the oracle's loop restarts the episode with
    # a branch and stops it there.  Every output the oracle makes non-finite is
    # non-finite here, the others lie in rows with a non-finite input on the
    # near side of them, and every output finite on both sides matches.
    p = params32(DEFAULT_PARAMS)
    N, T = 16, 700
    host = random_inputs(algo, N, T, 1200, dtype, p_term=0.01, p_trunc=0.005)
    r = host["rewards"].clone()
    bad = {3: 500, 7: 10, 11: 350, 12: 699}
    for row, col in bad.items():
        r[row, col] = float("inf") if row == 11 else float("nan")
    host["rewards"] = r
    got = run_gpu(algo, to_device(host), p)
    ref = run_oracle(algo, host, p)
    forward = algo in FORWARD
    for k in ref:
        gn, rn = ~np.isfinite(got[k]), ~np.isfinite(ref[k])
        assert np.all(gn[rn]), (k, "the oracle's non-finite outputs must be non-finite")
        for row, col in np.argwhere(gn & ~rn):
            assert row in bad, (k, row, col)
            # V-trace's pg reads the next step's vs: one step past the input
            assert (col >= bad[row]) if forward else (col <= bad[row] + 1), (k, row, col)
        fin = ~gn
        assert rel_err(got[k][fin], ref[k][fin]) <= TOL[dtype], k
    # the NaN of row 3 reaches every step on its far side, boundaries included
    first = got[next(iter(ref))][3]
    assert np.isnan(first[500:] if forward else first[:501]).all()
