"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/rlca.h declares, and rejects bad arguments with the documented
status before anything is enqueued (validation makes no HIP call).

The arrays here are fake device addresses that nothing may dereference, so
every call in this file must fail validation: a call that passed it would
enqueue a kernel on those addresses.  The one check that needs a call to pass
validation (adjacent arrays do not alias) runs only where no GPU is present,
where the launch itself fails (RLCA_EHIP)."""
import ctypes
import math
import os
import re

import pytest
import torch

import reverse_linear_recurrence_amd as rl
from split_rules import chain_segments
from reverse_linear_recurrence_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlca.h")

# Every array here is a fake address: should a call pass validation where a
# GPU is present, it would enqueue a kernel on them.  The module runs only
# where none is (the library then fails any launch with RLCA_EHIP).
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake device addresses: run where no GPU is present")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlca_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return rl.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_binding._SIGNATURES), "binding and header disagree"


def test_version_and_variants(lib):
    assert rl.rlca_version() >= 100
    nv = rl.rlca_num_variants()
    assert nv == 9
    for v in range(nv):
        for algo in rl.ALGO_CODES:
            k, lpr, wpr = rl.rlca_variant_info(v, torch.float32, algo)
            kb, lprb, wprb = rl.rlca_variant_info(v, torch.bfloat16, algo)
            assert k == 4  # one 16-byte fp32 vector per lane and array
            # bf16: one 16-byte vector per lane in the wide variants 6-8
            # (V-trace keeps 4 steps), 4 steps elsewhere
            assert kb == (8 if v >= 6 and algo != "vtrace" else 4)
            assert (lpr, wpr) == (lprb, wprb)
            if v >= 6:  # the wide twins of variants 3-5
                assert (lpr, wpr) == rl.rlca_variant_info(v - 3, torch.float32, algo)[1:]
            # lanes that share a row: part of a wavefront, or whole wavefronts
            assert (wpr == 1 and lpr in (16, 32, 64)) or lpr == 64 * wpr
    with pytest.raises(rl.RlcaError):
        rl.rlca_variant_info(nv)
    with pytest.raises(ValueError):
        rl.rlca_variant_info(0, torch.float32, "sarsa")
    lib = rl.load_library()
    k = ctypes.c_int()
    assert lib.rlca_variant_info(0, 8, 0, ctypes.byref(k), None, None) == rl.RLCA_EINVAL
    assert lib.rlca_variant_info(0, -1, 0, ctypes.byref(k), None, None) == rl.RLCA_EINVAL
    assert rl.rlca_set_variant(2) == -1
    assert rl.rlca_set_variant(-1) == 2
    with pytest.raises(ValueError):
        rl.rlca_set_variant(nv)
    assert rl.rlca_set_variant(-1) == -1


# Fake, never-dereferenced device addresses: validation fails before launch.
BASE = 0x7F0000000000
R, V, TE, TR, TV, ADV, TGT = (BASE + i * 0x1000000 for i in range(7))
F32 = 0


def gae(lib, N=4, T=8, dtype=F32, r=R, ld_r=None, v=V, ld_v=None, te=TE, tr=TR, tv=TV,
        ld_f=None, gamma=0.99, lam=0.95, adv=ADV, ld_a=None, tgt=TGT, ld_g=None):
    ld_r = T if ld_r is None else ld_r
    ld_v = T + 1 if ld_v is None else ld_v
    ld_f = T if ld_f is None else ld_f
    ld_a = T if ld_a is None else ld_a
    ld_g = T if ld_g is None else ld_g
    return lib.rlca_gae(N, T, dtype, r, ld_r, v, ld_v, te, ld_f, tr, ld_f, tv, ld_f,
                        gamma, lam, adv, ld_a, tgt, ld_g, None)


def err(lib):
    return lib.rlca_last_error().decode()


def test_empty_inputs_are_ok_without_launch(lib):
    assert gae(lib, N=0) == rl.RLCA_OK
    # Nothing is read or written for an empty batch, so no pointer is needed.
    assert gae(lib, N=0, r=None, v=None, adv=None) == rl.RLCA_OK
    # Parameters are still validated.
    assert gae(lib, N=0, gamma=3.0) == rl.RLCA_EINVAL


def test_rows_without_steps_are_rejected(lib):
    # T < 1 is an error, with or without rows.
    for N in (0, 4):
        assert gae(lib, N=N, T=0) == rl.RLCA_EINVAL
        assert "T = 0 must be >= 1" in err(lib)
    assert lib.rlca_returns(4, 0, 0, R, 8, None, 8, None, 8, None, 8, None, 0.9,
                            ADV, 8, None) == rl.RLCA_EINVAL
    assert lib.rlca_affine_scan(0, 0, F32, R, 8, V, 8, None, 8, 1, None, ADV, 8, None, None,
                                None, 0, None) == rl.RLCA_EINVAL
    assert lib.rlca_retrace_probs(4, 0, 5, F32, R, 8, V, 45, TE, 8, TR, 45, TV, 40, 0, None, 8,
                                  None, 8, None, 8, 0.9, 0.9, 1.0, ADV, 8, None) == rl.RLCA_EINVAL
    assert "T = 0" in err(lib)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=-1), rl.RLCA_EINVAL, "num_envs"),
    (dict(T=-3), rl.RLCA_EINVAL, "T ="),
    (dict(N=2 ** 31), rl.RLCA_EINVAL, "2^31"),
    (dict(dtype=7), rl.RLCA_EDTYPE, "dtype"),
    (dict(r=None), rl.RLCA_EINVAL, "rewards must not be NULL"),
    (dict(v=None), rl.RLCA_EINVAL, "values must not be NULL"),
    (dict(adv=None), rl.RLCA_EINVAL, "advantages must not be NULL"),
    (dict(tv=None), rl.RLCA_EINVAL, "trunc_values is NULL"),
    (dict(ld_r=7), rl.RLCA_EINVAL, "ld_rewards"),
    (dict(ld_v=8), rl.RLCA_EINVAL, "ld_values"),
    (dict(ld_f=5), rl.RLCA_EINVAL, "ld_terminated"),
    (dict(ld_a=1), rl.RLCA_EINVAL, "ld_advantages"),
    (dict(r=R + 2), rl.RLCA_EINVAL, "aligned"),
    (dict(adv=ADV + 1), rl.RLCA_EINVAL, "aligned"),
    (dict(gamma=1.5), rl.RLCA_EINVAL, "gamma"),
    (dict(gamma=-0.1), rl.RLCA_EINVAL, "gamma"),
    (dict(gamma=math.nan), rl.RLCA_EINVAL, "gamma"),
    (dict(lam=math.nan), rl.RLCA_EINVAL, "lam"),
    (dict(lam=1.01), rl.RLCA_EINVAL, "lam"),
    (dict(ld_r=2 ** 31), rl.RLCA_EINVAL, "exceeds 2^31-1"),
    (dict(N=2 ** 31 - 1, ld_r=2 ** 31 - 1, ld_v=2 ** 31 - 1, ld_f=2 ** 31 - 1,
          ld_a=2 ** 31 - 1, ld_g=2 ** 31 - 1), rl.RLCA_EINVAL, "overflow"),
    (dict(T=2 ** 31 - 1), rl.RLCA_EINVAL, "2^31-2"),
])
def test_gae_rejects_bad_arguments(lib, kw, status, needle):
    assert gae(lib, **kw) == status
    assert needle in err(lib)


def test_aliasing_is_rejected(lib):
    # advantages overlapping rewards, targets overlapping advantages, the last
    # element of a strided output overlapping an input's first element.
    assert gae(lib, adv=R + 4 * 4) == rl.RLCA_EALIAS
    assert "advantages" in err(lib) and "rewards" in err(lib)
    assert gae(lib, tgt=ADV + 4 * 5) == rl.RLCA_EALIAS
    assert "targets" in err(lib)
    span = (4 - 1) * 8 + 8  # elements of a [4, 8] array
    assert gae(lib, adv=R - span * 4 + 4) == rl.RLCA_EALIAS


def test_adjacent_arrays_do_not_alias(lib):
    # Passing validation enqueues a kernel on the fake addresses; with no GPU
    # present (the module's condition) the launch itself fails.
    span = (4 - 1) * 8 + 8
    assert gae(lib, adv=R - span * 4) == rl.RLCA_EHIP  # adjacent, not overlapping
    assert "launch" in err(lib)


def test_truncation_without_flags_needs_no_trunc_values(lib):
    # truncated == NULL: trunc_values is ignored; validation then proceeds to
    # the launch, which fails without a GPU (EHIP) or succeeds with one.
    rc = gae(lib, tr=None, tv=None, N=0)
    assert rc == rl.RLCA_OK


def test_other_entry_points_validate(lib):
    assert lib.rlca_returns(4, 8, 0, None, 8, None, 8, None, 8, None, 8, None, 0.9,
                            ADV, 8, None) == rl.RLCA_EINVAL
    assert lib.rlca_returns(4, 8, 0, R, 8, None, 8, None, 8, None, 8, None, 1.5,
                            ADV, 8, None) == rl.RLCA_EINVAL
    # bootstrap overlapping the output
    assert lib.rlca_returns(4, 8, 0, R, 8, None, 8, None, 8, None, 8, ADV + 8, 0.9,
                            ADV, 8, None) == rl.RLCA_EALIAS
    assert lib.rlca_td_lambda(4, 8, 0, R, 8, V, 8, None, 8, None, 8, None, 8, 0.9, 0.9,
                              ADV, 8, None) == rl.RLCA_EINVAL  # ld_values < T+1
    assert "ld_values" in err(lib)
    vt = lambda **k: lib.rlca_vtrace(4, 8, 0, R, 8, V, 9, k.get("lr", TE), 8, None, 8, None, 8,
                                      None, 8, 0.9, 0.9, k.get("rho", 1.0), k.get("c", 1.0),
                                      k.get("pg", 1.0), ADV, 8, k.get("pgp", None), 8, None)
    assert vt(rho=0.0) == rl.RLCA_EINVAL and "rho_bar" in err(lib)
    assert vt(c=-1.0) == rl.RLCA_EINVAL and "c_bar" in err(lib)
    assert vt(pg=math.nan) == rl.RLCA_EINVAL and "pg_rho_bar" in err(lib)
    assert vt(lr=None) == rl.RLCA_EINVAL and "log_rhos" in err(lib)
    assert vt(pgp=ADV) == rl.RLCA_EALIAS
    rt = lambda **k: lib.rlca_retrace(4, 8, 0, R, 8, k.get("q", V), 8, k.get("eq", TV), 8, TE,
                                       8, None, 8, None, 8, 0.9, 0.9, k.get("c", 1.0),
                                       k.get("out", ADV), 8, None)
    assert rt(q=None) == rl.RLCA_EINVAL and "q_taken" in err(lib)
    assert rt(eq=None) == rl.RLCA_EINVAL and "exp_q_next" in err(lib)
    assert rt(c=0.0) == rl.RLCA_EINVAL
    assert rt(out=TV + 4) == rl.RLCA_EALIAS and "exp_q_next" in err(lib)


def test_error_message_is_per_thread(lib):
    import threading
    assert gae(lib, gamma=2.0) == rl.RLCA_EINVAL
    seen = {}

    def other():
        seen["msg"] = lib.rlca_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "gamma" in err(lib)


def test_binding_refuses_cpu_tensors():
    r = torch.zeros(2, 4)
    v = torch.zeros(2, 5)
    with pytest.raises(ValueError, match="GPU"):
        rl.rlca_gae(r, v, gamma=0.9, lam=0.9)
    with pytest.raises(ValueError, match="2-D"):
        rl.rlca_returns(torch.zeros(4), gamma=0.9)


# Window entry points: the carry vectors are validated like every array.
C_IN, C_OUT, C_MAP = (BASE + (8 + i) * 0x1000000 for i in range(3))


def gae_chunk(lib, N=4, T=8, cin=C_IN, cout=C_OUT, cmap=C_MAP, adv=ADV, r=R, ws=None,
              ws_bytes=0):
    return lib.rlca_gae_chunk(N, T, F32, r, T, V, T + 1, TE, T, TR, T, TV, T, 0.9, 0.9,
                              adv, T, TGT, T, cin, cout, cmap, ws, ws_bytes, None)


def test_window_entry_points_validate_carry_vectors(lib):
    assert gae_chunk(lib, N=0) == rl.RLCA_OK
    assert gae_chunk(lib, cin=C_IN + 2) == rl.RLCA_EINVAL and "carry_in" in err(lib)
    assert gae_chunk(lib, cout=C_OUT + 1) == rl.RLCA_EINVAL and "carry_out" in err(lib)
    # carry_out overlapping carry_in (no in-place update), carry_map
    # overlapping carry_out, a carry output overlapping an input array.
    assert gae_chunk(lib, cout=C_IN + 4) == rl.RLCA_EALIAS and "carry_in" in err(lib)
    assert gae_chunk(lib, cout=C_IN) == rl.RLCA_EALIAS
    assert gae_chunk(lib, cmap=C_OUT + 12) == rl.RLCA_EALIAS and "carry_map" in err(lib)
    assert gae_chunk(lib, cmap=R + 8) == rl.RLCA_EALIAS and "rewards" in err(lib)
    # The map holds 2 floats per row: one float past the carry vector's end
    # is still an overlap for the map, not for the carry.
    assert gae_chunk(lib, cmap=C_OUT - 2 * 4 * 4 + 4) == rl.RLCA_EALIAS
    ret = lambda **k: lib.rlca_returns_chunk(4, 8, F32, R, 8, None, 8, None, 8, None, 8,
                                              k.get("cin", C_IN), k.get("gamma", 0.9), ADV, 8,
                                              k.get("cout", C_OUT), None, None, 0, None)
    assert ret(gamma=1.5) == rl.RLCA_EINVAL
    assert ret(cout=ADV + 4) == rl.RLCA_EALIAS
    el = lambda **k: lib.rlca_eligibility_trace_chunk(4, 8, F32, R, 8, None, 8, None, 8,
                                                       k.get("cin", C_IN), 0.9, k.get("lam", 0.9),
                                                       ADV, 8, C_OUT, C_MAP, None, 0, None)
    assert el(lam=2.0) == rl.RLCA_EINVAL and "lam" in err(lib)
    assert el(cin=ADV) == rl.RLCA_EALIAS


def test_affine_scan_validates(lib):
    aff = lambda **k: lib.rlca_affine_scan(k.get("N", 4), 8, k.get("dtype", F32), k.get("a", R),
                                           8, k.get("b", V), 8, k.get("rs", None), 8,
                                           k.get("rev", 1), None, k.get("out", ADV), 8, None,
                                           None, None, 0, None)
    assert aff(N=0) == rl.RLCA_OK
    assert aff(rev=2) == rl.RLCA_EINVAL and "reverse" in err(lib)
    assert aff(b=None) == rl.RLCA_EINVAL and "beta" in err(lib)
    assert aff(a=None) == rl.RLCA_EINVAL and "alpha" in err(lib)
    assert aff(out=None) == rl.RLCA_EINVAL and "out" in err(lib)
    assert aff(dtype=5) == rl.RLCA_EDTYPE
    assert aff(out=V + 4) == rl.RLCA_EALIAS and "beta" in err(lib)
    assert aff(rs=ADV + 3) == rl.RLCA_EALIAS and "reset" in err(lib)


def test_binding_refuses_bad_carry_vectors():
    with pytest.raises(ValueError, match="GPU"):
        rl.rlca_affine_scan(torch.zeros(2, 4), torch.zeros(2, 4))


def test_policy_table_entry_points_validate(lib):
    Q, ACT, LP, LM = (BASE + (12 + i) * 0x1000000 for i in range(4))
    rp = lambda **k: lib.rlca_retrace_probs(
        4, 8, k.get("A", 5), F32, R, 8, k.get("q", Q), k.get("ld_q", 45), k.get("act", ACT), 8,
        LP, k.get("ld_lp", 45), LM, k.get("ld_lm", 40), k.get("taken", 0), None, 8,
        k.get("tr", None), 8,
        k.get("teq", None), 8, 0.9, 0.9, 1.0, k.get("out", ADV), 8, None)
    assert rp(A=0) == rl.RLCA_EINVAL and "num_actions" in err(lib)
    assert rp(A=65537) == rl.RLCA_EINVAL
    assert rp(ld_q=44) == rl.RLCA_EINVAL and "ld_q_values" in err(lib)   # needs (T+1)*A
    assert rp(ld_lp=40) == rl.RLCA_EINVAL and "ld_log_pi" in err(lib)
    assert rp(ld_lm=39) == rl.RLCA_EINVAL and "ld_log_mu" in err(lib)
    assert rp(taken=2) == rl.RLCA_EINVAL and "log_mu_taken" in err(lib)
    assert rp(ld_lm=7, taken=1) == rl.RLCA_EINVAL and "ld_log_mu" in err(lib)
    assert rp(act=ACT + 2) == rl.RLCA_EINVAL and "actions" in err(lib)
    assert rp(q=None) == rl.RLCA_EINVAL and "q_values" in err(lib)
    assert rp(tr=TR) == rl.RLCA_EINVAL and "trunc_eq" in err(lib)
    assert rp(out=Q + 4) == rl.RLCA_EALIAS and "q_values" in err(lib)
    vt = lambda **k: lib.rlca_vtrace_probs(
        4, 8, 5, F32, R, 8, V, 9, ACT, 8, LP, k.get("ld_lp", 40), LM, 40, 0, None, 8, None, 8,
        None, 8, 0.9, 0.9, k.get("rho", 1.0), 1.0, 1.0, ADV, 8, k.get("pg", None), 8, None)
    assert vt(ld_lp=39) == rl.RLCA_EINVAL and "ld_log_pi" in err(lib)
    assert vt(rho=0.0) == rl.RLCA_EINVAL and "rho_bar" in err(lib)
    assert vt(pg=ACT) == rl.RLCA_EALIAS and "actions" in err(lib)


def test_policy_table_window_entry_points_validate(lib):
    # The window forms check their per-row carry vectors like rlca_gae_chunk.
    Q, ACT, LP, LM = (BASE + (12 + i) * 0x1000000 for i in range(4))
    rpc = lambda **k: lib.rlca_retrace_probs_chunk(
        k.get("N", 4), 8, 5, F32, R, 8, Q, 45, ACT, 8, LP, 45, LM, 40, 0, None, 8, None, 8,
        None, 8, 0.9, 0.9, 1.0, ADV, 8, k.get("cin", C_IN), k.get("cout", C_OUT),
        k.get("cmap", C_MAP), None)
    assert rpc(N=0) == rl.RLCA_OK
    assert rpc(cin=C_IN + 2) == rl.RLCA_EINVAL and "carry_in" in err(lib)
    assert rpc(cout=C_OUT + 1) == rl.RLCA_EINVAL and "carry_out" in err(lib)
    assert rpc(cout=C_IN) == rl.RLCA_EALIAS and "carry_in" in err(lib)
    assert rpc(cmap=Q + 8) == rl.RLCA_EALIAS and "q_values" in err(lib)
    assert rpc(cmap=ADV) == rl.RLCA_EALIAS
    vtc = lambda **k: lib.rlca_vtrace_probs_chunk(
        k.get("N", 4), 8, 5, F32, R, 8, V, 9, ACT, 8, LP, 40, LM, 40, 0, None, 8, None, 8,
        None, 8, 0.9, 0.9, 1.0, 1.0, 1.0, ADV, 8, None, 8, k.get("cin", C_IN),
        k.get("cout", C_OUT), k.get("cmap", C_MAP), None)
    assert vtc(N=0) == rl.RLCA_OK
    assert vtc(cmap=C_MAP + 2) == rl.RLCA_EINVAL and "carry_map" in err(lib)
    assert vtc(cout=LP + 16) == rl.RLCA_EALIAS and "log_pi" in err(lib)
    assert vtc(cmap=C_OUT) == rl.RLCA_EALIAS and "carry_out" in err(lib)


def test_split_segments_rule(lib):
    # the smallest power of two S with N * S >= 256, T % S == 0 and
    # T / S >= 4096, stopping where either would fail; no split above 64 rows
    # or below 32768 steps per row
    cases = {(64, 65536): 4, (16, 262144): 16, (1, 32768): 8, (1, 1 << 20): 256,
             (2, 1 << 19): 128, (3, 32768): 8, (65, 65536): 1, (127, 65536): 1,
             (128, 32768): 1, (3, 16384): 1, (100, 16384): 1, (8, 4096): 1, (2, 3 * 16384): 8,
             (2, 32769): 1, (2, 2 * 32769): 2, (0, 1): 1}
    for (N, T), S in cases.items():
        assert rl.rlca_split_segments(N, T) == S, (N, T)
        chained = max(8 + 32 * N * chain_segments(N, T, dt, algo) if chain_segments(
            N, T, dt, algo) else 0 for dt in (torch.float32, torch.bfloat16)
            for algo in rl.ALGO_CODES)
        assert rl.rlca_split_workspace_bytes(N, T) == max(12 * N * S if S > 1 else 0,
                                                          chained), (N, T)
    # the chained form's segments: one or two whole tiles of a whole-wavefront
    # tiling, at most 256 per row, the least
    # ceil(N * S / 256) * L + ceil(N * S / (256 * r)) * 4096 + 32 * S
    assert chain_segments(16, 262144, torch.float32, "gae") == 32  # 2 tiles of 4096
    assert chain_segments(16, 262144, torch.bfloat16, "gae") == 16  # 2 tiles of 8192
    assert chain_segments(64, 65536, torch.bfloat16, "gae") == 4
    assert chain_segments(1, 32768, torch.float32, "gae") == 32  # 1 tile of 1024
    assert chain_segments(1, 1 << 20, torch.bfloat16, "gae") == 128  # 1 tile of 8192
    assert chain_segments(1, 1 << 21, torch.float32, "gae") == 256  # 2 tiles of 4096
    assert chain_segments(1, 1 << 22, torch.float32, "gae") == 0  # 512 segments at least
    assert chain_segments(65, 65536, torch.float32, "gae") == 8  # 2 tiles of 4096 (tie: longer)
    assert chain_segments(160, 32768, torch.bfloat16, "gae") == 4  # 1 tile of 8192 (tie)
    assert chain_segments(224, 32768, torch.bfloat16, "gae") == 2  # 2 tiles of 8192
    assert chain_segments(225, 65536, torch.bfloat16, "gae") == 0
    assert chain_segments(128, 16384, torch.bfloat16, "gae") == 2  # N <= T / 128
    assert chain_segments(129, 16384, torch.bfloat16, "gae") == 0
    assert chain_segments(16, 8192, torch.bfloat16, "gae") == 4  # 1 tile of 2048
    assert chain_segments(64, 8192, torch.float32, "gae") == 4  # segments of 2048 steps
    assert chain_segments(32, 4096, torch.bfloat16, "gae") == 0  # T < 8192
    assert chain_segments(100, 32768, torch.float32, "vtrace") == 4
    assert chain_segments(2, 32769, torch.float32, "gae") == 0
    assert chain_segments(8, 32768, torch.bfloat16, "gae") == 16  # wide: 1 tile of 2048
    assert chain_segments(1, 33 * 1024, torch.bfloat16, "gae") == 33  # no wide tile divides T
    assert chain_segments(1, 33 * 1024, torch.bfloat16, "vtrace") == 33
    # the three-launch form: at most 64 rows, fewer than 512 segments in all
    assert max(N * rl.rlca_split_segments(N, 1 << 24) for N in range(1, 65)) < 512
    for bad in ((-1, 8), (4, 0)):
        with pytest.raises(ValueError):
            rl.rlca_split_segments(*bad)
        with pytest.raises(ValueError):
            rl.rlca_split_workspace_bytes(*bad)
    assert lib.rlca_split_segments(4, -8) == -1 and "T" in err(lib)
    assert lib.rlca_split_workspace_bytes(4, 0) == -1 and "T >= 1" in err(lib)


WS = BASE + 0x40000000  # a fake workspace clear of every array above


def test_workspace_is_validated(lib):
    # A window call that splits (16 rows of 65536 steps: 16 segments each)
    # checks its 3 * 16 * 16 floats of workspace before any launch.
    N, T = 16, 65536
    need = rl.rlca_split_workspace_bytes(N, T)
    assert need == 8 + 32 * N * 16  # the chained form's, above the three-launch form's
    assert gae_chunk(lib, N=N, T=T, ws=WS + 2, ws_bytes=need) == rl.RLCA_EINVAL
    assert "aligned" in err(lib)
    assert gae_chunk(lib, N=N, T=T, ws=WS, ws_bytes=-4) == rl.RLCA_EINVAL
    assert "negative" in err(lib)
    # below what the three-launch form needs (a size that fits only that form
    # selects it)
    assert gae_chunk(lib, N=N, T=T, ws=WS, ws_bytes=12 * N * 16 - 4) == rl.RLCA_EINVAL
    assert "rlca_split_workspace_bytes" in err(lib)
    # overlapping an output, an input
    assert gae_chunk(lib, N=N, T=T, ws=ADV + 64, ws_bytes=need) == rl.RLCA_EALIAS
    assert "workspace" in err(lib)
    assert gae_chunk(lib, N=N, T=T, ws=R + 4 * 65536 * 16 - 8, ws_bytes=need) == rl.RLCA_EALIAS
    assert "rewards" in err(lib)
    with pytest.raises(ValueError):
        rl.rlca_affine_scan(torch.zeros(2, 4), torch.zeros(2, 4),
                            workspace=torch.empty(16))  # not on a GPU


def test_split_window_call_validates_its_workspace(lib):
    # A window call that splits checks the window's three carry vectors and
    # the workspace, all beside its own arrays (the argument table has room
    # for four more entries), before any launch.
    N, T = 16, 65536
    need = rl.rlca_split_workspace_bytes(N, T)
    for _ in range(3):
        assert gae_chunk(lib, N=N, T=T, r=R, ws=R + 64, ws_bytes=need) == rl.RLCA_EALIAS
        assert "workspace" in err(lib)
        assert lib.rlca_returns_chunk(N, T, F32, R, T, None, T, None, T, None, T, C_IN, 0.9,
                                      ADV, T, C_OUT, C_MAP, R + 64, need,
                                      None) == rl.RLCA_EALIAS
        assert lib.rlca_affine_scan(N, T, F32, R, T, V, T, None, T, 0, C_IN, ADV, T, C_OUT,
                                    C_MAP, V + 8, need, None) == rl.RLCA_EALIAS
        assert "workspace" in err(lib)
    assert gae_chunk(lib, N=N, T=T, ws=C_MAP + 8, ws_bytes=need) == rl.RLCA_EALIAS
    assert "carry_map" in err(lib)
    # the carry vectors are validated when a workspace is given too
    assert gae_chunk(lib, N=N, T=T, cin=C_IN + 2, ws=WS, ws_bytes=need) == rl.RLCA_EINVAL
    assert "carry_in" in err(lib)


def test_materialized_scan_validates_its_workspace(lib):
    # The materialized doubling scan needs 16 bytes per step of workspace,
    # checked (with the call's own arrays) before any launch.
    N, T = 4, 8
    need = rl.rlca_materialized_workspace_bytes(N, T)
    assert need == 16 * N * T
    assert rl.rlca_materialized_workspace_bytes(0, 5) == 0
    with pytest.raises(ValueError):
        rl.rlca_materialized_workspace_bytes(2, 0)
    assert lib.rlca_materialized_workspace_bytes(2 ** 31 - 1, 2 ** 31 - 2) == -1

    def g(ws, nb, **k):
        return lib.rlca_gae_materialized(k.get("N", N), T, F32, R, T, V, T + 1, TE, T, TR, T, TV,
                                         T, k.get("gamma", 0.9), 0.9, ADV, T, TGT, T, ws, nb,
                                         None)
    assert g(None, 0) == rl.RLCA_EINVAL and "needs a workspace" in err(lib)
    assert g(WS, need - 4) == rl.RLCA_EINVAL and "rlca_materialized_workspace_bytes" in err(lib)
    assert g(WS + 2, need) == rl.RLCA_EINVAL and "aligned" in err(lib)
    assert g(WS, -1) == rl.RLCA_EINVAL
    assert g(ADV + 16, need) == rl.RLCA_EALIAS and "workspace" in err(lib)
    assert g(V + 8, need) == rl.RLCA_EALIAS and "values" in err(lib)
    assert g(WS, need, gamma=2.0) == rl.RLCA_EINVAL and "gamma" in err(lib)
    assert g(None, 0, N=0) == rl.RLCA_EINVAL  # the workspace is required, rows or not
    assert g(WS, need, N=0) == rl.RLCA_OK
    rt = lib.rlca_retrace_materialized(N, T, F32, R, T, V, T, TV, T, TE, T, None, T, None, T,
                                       0.9, 0.9, 0.0, ADV, T, WS, need, None)
    assert rt == rl.RLCA_EINVAL and "c_bar" in err(lib)
    vt = lib.rlca_vtrace_materialized(N, T, F32, R, T, V, T + 1, TE, T, None, T, None, T, None,
                                      T, 0.9, 0.9, 1.0, 1.0, 1.0, ADV, T, R, T, WS, need, None)
    assert vt == rl.RLCA_EALIAS and "pg_advantages" in err(lib)
    ret = lib.rlca_returns_materialized(N, T, F32, R, T, None, T, None, T, None, T,
                                        WS + need - 4, 0.9, ADV, T, WS, need, None)
    assert ret == rl.RLCA_EALIAS and "bootstrap" in err(lib)
