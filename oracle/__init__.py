"""fp64 CPU oracle for reverse-time credit-assignment recurrences.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product path (``reverse_linear_recurrence_amd``) never imports
it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one backward
loop per row); this module only marshals numpy arrays into it.  Every function
takes row-major arrays, widens all floating-point inputs to float64 (exactly:
bf16 and fp32 values are representable), and returns float64 arrays.

Flags are ``uint8``/``bool`` arrays of shape ``[N, T]``; ``None`` means "never".
``values`` has shape ``[N, T+1]``: column ``T`` is the window-end bootstrap.
``trunc_values`` ``[N, T]`` is read only where a truncation is not also a
termination (termination wins).

Window carries: ``carry_in [N]`` (None: 0) is the scan state just past the
window end (reverse recurrences; ``bootstrap`` for returns) or just before its
start (forward ones; ``z_init`` / ``s_init``).  With ``chunk=True`` a function
also returns ``carry_out [N]`` (the neighbouring window's carry_in) and
``carry_map [N, 2]`` = (a, b) with carry_out = a + b * carry_in.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle, stale

_lib = None
_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is None:
        if stale():
            build_oracle()
        lib = ctypes.CDLL(LIB)
        i64, dbl = ctypes.c_int64, ctypes.c_double
        lib.oracle_returns.argtypes = [i64, i64, _D, _U8, _U8, _D, _D, dbl, _D, _D, _D]
        lib.oracle_gae.argtypes = [i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D, _D,
                                   _D, _D, _D]
        lib.oracle_td_lambda.argtypes = [i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D,
                                         _D, _D, _D]
        lib.oracle_vtrace.argtypes = [i64, i64, _D, _D, _D, _U8, _U8, _D,
                                      dbl, dbl, dbl, dbl, dbl, _D, _D, _D, _D, _D]
        lib.oracle_retrace.argtypes = [i64, i64, _D, _D, _D, _D, _U8, _U8,
                                       dbl, dbl, dbl, _D, _D, _D, _D]
        lib.oracle_eligibility_trace.argtypes = [i64, i64, _D, _U8, _U8, _D, dbl, dbl, _D,
                                                 _D, _D]
        lib.oracle_episodic_cumsum.argtypes = [i64, i64, _D, _U8, _U8, _D, _D, _D, _D]
        lib.oracle_affine_scan.argtypes = [i64, i64, _D, _D, _U8, ctypes.c_int, _D,
                                           _D, _D, _D]
        _I32 = ctypes.POINTER(ctypes.c_int32)
        ci = ctypes.c_int
        lib.oracle_retrace_probs.argtypes = [i64, i64, i64, _D, _D, _I32, _D, _D, ci, _U8, _U8,
                                             _D, dbl, dbl, dbl, _D, _D, _D, _D]
        lib.oracle_vtrace_probs.argtypes = [i64, i64, i64, _D, _D, _I32, _D, _D, ci, _U8, _U8,
                                            _D, dbl, dbl, dbl, dbl, dbl, _D, _D, _D, _D, _D]
        for f in (lib.oracle_returns, lib.oracle_gae, lib.oracle_td_lambda,
                  lib.oracle_vtrace, lib.oracle_retrace, lib.oracle_eligibility_trace,
                  lib.oracle_episodic_cumsum, lib.oracle_affine_scan,
                  lib.oracle_retrace_probs, lib.oracle_vtrace_probs):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x, shape):
    if x is None:
        return None, None
    a = np.ascontiguousarray(_as_numpy(x), dtype=np.float64)
    if a.shape != shape:
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a, a.ctypes.data_as(_D)


def _u8(x, shape):
    if x is None:
        return None, None
    a = np.ascontiguousarray(_as_numpy(x)).astype(np.uint8, copy=False)
    if a.shape != shape:
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a, a.ctypes.data_as(_U8)


def _as_numpy(x):
    # torch tensors (including bfloat16) are accepted without importing torch here.
    if hasattr(x, "detach") and hasattr(x, "float"):
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        return x.numpy()
    return np.asarray(x)


def _check(rc, name):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % name)


class _Carry:
    """carry_out [N] and carry map [N, 2] buffers of one call."""

    def __init__(self, N):
        self.out = np.empty(N, np.float64)
        self.map = np.empty((N, 2), np.float64)
        self.out_p = self.out.ctypes.data_as(_D)
        self.map_p = self.map.ctypes.data_as(_D)


def returns(rewards, terminated=None, truncated=None, trunc_values=None,
            bootstrap=None, *, gamma, chunk=False):
    """Discounted returns ``G [N, T]``; ``bootstrap [N]`` is the carry ``G_T`` (None: 0).

    chunk=True: ``(G, carry_out, carry_map)``, carry_out = G_0."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    b, bp = _f64(bootstrap, (N,))
    out = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_returns(N, T, rp, tep, trp, tvp, bp, float(gamma),
                                  out.ctypes.data_as(_D), c.out_p, c.map_p), "returns")
    return (out, c.out, c.map) if chunk else out


def gae(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
        gamma, lam, carry_in=None, chunk=False):
    """GAE: returns ``(advantages, targets)``, each ``[N, T]``.

    carry_in: A_T (advantage of the step after the window).  chunk=True adds
    ``carry_out`` (= A_0) and ``carry_map``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    adv = np.empty((N, T), np.float64)
    tgt = np.empty((N, T), np.float64)
    ci, cip = _f64(carry_in, (N,))
    c = _Carry(N)
    _check(_load().oracle_gae(N, T, rp, vp, tep, trp, tvp, float(gamma), float(lam),
                              adv.ctypes.data_as(_D), tgt.ctypes.data_as(_D), cip, c.out_p,
                              c.map_p), "gae")
    return (adv, tgt, c.out, c.map) if chunk else (adv, tgt)


def td_lambda(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
              gamma, lam, carry_in=None, chunk=False):
    """TD(lambda) returns ``[N, T]``.

    carry_in: G_T - V_T of the step after the window.  chunk=True adds
    ``carry_out`` (= G_0 - V_0) and ``carry_map``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    out = np.empty((N, T), np.float64)
    ci, cip = _f64(carry_in, (N,))
    c = _Carry(N)
    _check(_load().oracle_td_lambda(N, T, rp, vp, tep, trp, tvp, float(gamma), float(lam),
                                    out.ctypes.data_as(_D), cip, c.out_p, c.map_p), "td_lambda")
    return (out, c.out, c.map) if chunk else out


def vtrace(rewards, values, log_rhos, terminated=None, truncated=None, trunc_values=None,
           *, gamma, lam, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0, carry_in=None,
           chunk=False):
    """V-trace: returns ``(vs, pg_advantages)``, each ``[N, T]``.

    carry_in: vs_T - V_T of the step after the window.  chunk=True adds
    ``carry_out`` (= vs_0 - V_0) and ``carry_map``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    lr, lrp = _f64(log_rhos, (N, T))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    vs = np.empty((N, T), np.float64)
    pg = np.empty((N, T), np.float64)
    ci, cip = _f64(carry_in, (N,))
    c = _Carry(N)
    _check(_load().oracle_vtrace(N, T, rp, vp, lrp, tep, trp, tvp, float(gamma), float(lam),
                                 float(rho_bar), float(c_bar), float(pg_rho_bar),
                                 vs.ctypes.data_as(_D), pg.ctypes.data_as(_D), cip, c.out_p,
                                 c.map_p), "vtrace")
    return (vs, pg, c.out, c.map) if chunk else (vs, pg)


def retrace(rewards, q_taken, exp_q_next, log_rhos, terminated=None, truncated=None, *,
            gamma, lam, c_bar=1.0, carry_in=None, chunk=False):
    """Retrace(lambda) targets ``Q^ret [N, T]``.

    carry_in: c_T * (Qret_T - Q_T) of the step after the window.  chunk=True
    adds ``carry_out`` (= c_0 * (Qret_0 - Q_0)) and ``carry_map``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    q, qp = _f64(q_taken, (N, T))
    eq, eqp = _f64(exp_q_next, (N, T))
    lr, lrp = _f64(log_rhos, (N, T))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    out = np.empty((N, T), np.float64)
    ci, cip = _f64(carry_in, (N,))
    c = _Carry(N)
    _check(_load().oracle_retrace(N, T, rp, qp, eqp, lrp, tep, trp, float(gamma), float(lam),
                                  float(c_bar), out.ctypes.data_as(_D), cip, c.out_p, c.map_p),
           "retrace")
    return (out, c.out, c.map) if chunk else out


def eligibility_trace(x, terminated=None, truncated=None, z_init=None, *, gamma, lam,
                      chunk=False):
    """Forward accumulating trace ``z [N, T]``: z_t = x_t + gamma*lam*(1-done_{t-1}) z_{t-1}.

    chunk=True adds ``carry_out`` (= z_{T-1}, 0 if done_{T-1}) and ``carry_map``."""
    a, ap = _f64(x, np.shape(_as_numpy(x)))
    N, T = a.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    z0, z0p = _f64(z_init, (N,))
    out = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_eligibility_trace(N, T, ap, tep, trp, z0p, float(gamma), float(lam),
                                            out.ctypes.data_as(_D), c.out_p, c.map_p),
           "eligibility_trace")
    return (out, c.out, c.map) if chunk else out


def episodic_cumsum(x, terminated=None, truncated=None, s_init=None, *, chunk=False):
    """Forward episodic prefix sum ``S [N, T]``: S_t = x_t + (1-done_{t-1}) S_{t-1}.

    chunk=True adds ``carry_out`` (= S_{T-1}, 0 if done_{T-1}) and ``carry_map``."""
    a, ap = _f64(x, np.shape(_as_numpy(x)))
    N, T = a.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    s0, s0p = _f64(s_init, (N,))
    out = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_episodic_cumsum(N, T, ap, tep, trp, s0p, out.ctypes.data_as(_D),
                                          c.out_p, c.map_p), "episodic_cumsum")
    return (out, c.out, c.map) if chunk else out


def affine_scan(alpha, beta, reset=None, carry_in=None, *, reverse=True):
    """Segmented affine scan ``A [N, T]`` with ``carry_out [N]`` and ``carry_map [N, 2]``.

    reverse: A_t = alpha_t + beta'_t A_{t+1} (A_T = carry_in); else
    A_t = alpha_t + beta'_t A_{t-1} (A_{-1} = carry_in); beta'_t = 0 where
    reset_t, else beta_t.  Returns ``(A, carry_out, carry_map)``."""
    a, ap = _f64(alpha, np.shape(_as_numpy(alpha)))
    N, T = a.shape
    b, bp = _f64(beta, (N, T))
    rs, rsp = _u8(reset, (N, T))
    ci, cip = _f64(carry_in, (N,))
    out = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_affine_scan(N, T, ap, bp, rsp, 1 if reverse else 0, cip,
                                      out.ctypes.data_as(_D), c.out_p, c.map_p), "affine_scan")
    return out, c.out, c.map


def _i32(x, shape):
    a = np.ascontiguousarray(_as_numpy(x)).astype(np.int32, copy=False)
    if a.shape != shape:
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def retrace_probs(rewards, q_values, actions, log_pi, log_mu, terminated=None, truncated=None,
                  trunc_eq=None, *, gamma, lam, c_bar=1.0, carry_in=None, chunk=False):
    """Retrace(lambda) from tables: q_values and log_pi ``[N, T+1, A]``,
    log_mu ``[N, T, A]`` (or ``[N, T]``: the taken actions' entries only),
    actions ``[N, T]``; trunc_eq ``[N, T]`` is E_pi Q at the true final state
    of truncated steps.  Returns ``Q^ret`` (chunk=True: also carry_out and
    carry_map)."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    A = np.shape(_as_numpy(q_values))[2]
    q, qp = _f64(q_values, (N, T + 1, A))
    ac, acp = _i32(actions, (N, T))
    lp, lpp = _f64(log_pi, (N, T + 1, A))
    mu_taken = len(np.shape(_as_numpy(log_mu))) == 2
    lm, lmp = _f64(log_mu, (N, T) if mu_taken else (N, T, A))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    te2, te2p = _f64(trunc_eq, (N, T))
    ci, cip = _f64(carry_in, (N,))
    out = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_retrace_probs(N, T, A, rp, qp, acp, lpp, lmp, int(mu_taken), tep,
                                        trp, te2p,
                                        float(gamma), float(lam), float(c_bar),
                                        out.ctypes.data_as(_D), cip, c.out_p, c.map_p),
           "retrace_probs")
    return (out, c.out, c.map) if chunk else out


def vtrace_probs(rewards, values, actions, log_pi, log_mu, terminated=None, truncated=None,
                 trunc_values=None, *, gamma, lam, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0,
                 carry_in=None, chunk=False):
    """V-trace from tables: log_pi and log_mu ``[N, T, A]`` (log_mu may be
    ``[N, T]``: the taken actions' entries only), actions ``[N, T]``.
    Returns ``(vs, pg_advantages)`` (chunk=True: also carry_out, carry_map)."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    A = np.shape(_as_numpy(log_pi))[2]
    v, vp = _f64(values, (N, T + 1))
    ac, acp = _i32(actions, (N, T))
    lp, lpp = _f64(log_pi, (N, T, A))
    mu_taken = len(np.shape(_as_numpy(log_mu))) == 2
    lm, lmp = _f64(log_mu, (N, T) if mu_taken else (N, T, A))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    ci, cip = _f64(carry_in, (N,))
    vs = np.empty((N, T), np.float64)
    pg = np.empty((N, T), np.float64)
    c = _Carry(N)
    _check(_load().oracle_vtrace_probs(N, T, A, rp, vp, acp, lpp, lmp, int(mu_taken), tep, trp,
                                       tvp,
                                       float(gamma), float(lam), float(rho_bar), float(c_bar),
                                       float(pg_rho_bar), vs.ctypes.data_as(_D),
                                       pg.ctypes.data_as(_D), cip, c.out_p, c.map_p),
           "vtrace_probs")
    return (vs, pg, c.out, c.map) if chunk else (vs, pg)


# ------------------------------------------------ the oracle on several threads
#
# The benchmark's CPU baseline times the oracle on every host core.  The C
# drivers of oracle_rows.c cut the rows into one contiguous slice per thread
# and run the unchanged serial functions above on each slice (OpenMP); one
# ctypes call covers a whole batch, with the interpreter lock released.

_ROWS_SIGS = None


def _rows_lib():
    global _ROWS_SIGS
    lib = _load()
    if _ROWS_SIGS is None:
        i64, dbl, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_int
        _I32 = ctypes.POINTER(ctypes.c_int32)
        sigs = {
            "returns": [ci, i64, i64, _D, _U8, _U8, _D, _D, dbl, _D],
            "gae": [ci, i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D, _D],
            "td_lambda": [ci, i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D],
            "vtrace": [ci, i64, i64, _D, _D, _D, _U8, _U8, _D, dbl, dbl, dbl, dbl, dbl, _D, _D],
            "retrace": [ci, i64, i64, _D, _D, _D, _D, _U8, _U8, dbl, dbl, dbl, _D],
            "eligibility_trace": [ci, i64, i64, _D, _U8, _U8, _D, dbl, dbl, _D],
            "episodic_cumsum": [ci, i64, i64, _D, _U8, _U8, _D, _D],
            "retrace_probs": [ci, i64, i64, i64, _D, _D, _I32, _D, _D, ci, _U8, _U8, _D, dbl,
                              dbl, dbl, _D],
            "vtrace_probs": [ci, i64, i64, i64, _D, _D, _I32, _D, _D, ci, _U8, _U8, _D, dbl,
                             dbl, dbl, dbl, dbl, _D, _D],
        }
        for name, argtypes in sigs.items():
            f = getattr(lib, "oracle_rows_" + name)
            f.argtypes = argtypes
            f.restype = ctypes.c_int
        lib.oracle_rows_threads.argtypes = []
        lib.oracle_rows_threads.restype = ctypes.c_int
        _ROWS_SIGS = sigs
    return lib


def batch_runner(algo, inputs, params, threads):
    """A function of no arguments that runs the oracle once over the whole
    batch ``inputs`` (a dict of the workload's arrays: rewards, values,
    terminated, ...) on ``threads`` host threads, one contiguous row slice
    each, and returns the list of its output arrays (float64 [N, T]; the
    same arrays on every call).  Arrays are widened and outputs allocated
    here, once.  ``algo`` is
    one of returns, gae, td_lambda, vtrace, retrace, eligibility_trace,
    episodic_cumsum, retrace_probs, vtrace_probs; ``params`` holds gamma, lam
    and the clips the algorithm takes."""
    lib = _rows_lib()
    g = inputs.get
    r, rp = _f64(g("rewards"), np.shape(_as_numpy(g("rewards"))))
    N, T = r.shape
    keep = [r]

    def f64(name, shape):
        a, p = _f64(g(name), shape)
        keep.append(a)
        return p

    def u8(name):
        a, p = _u8(g(name), (N, T))
        keep.append(a)
        return p

    outs = []

    def out():
        a = np.empty((N, T), np.float64)
        outs.append(a)
        return a.ctypes.data_as(_D)

    gamma = float(params["gamma"])
    lam = float(params.get("lam", 1.0))
    clips = [float(params.get(k, 1.0)) for k in ("rho_bar", "c_bar", "pg_rho_bar")]
    nt = int(threads)
    te, tr = u8("terminated"), u8("truncated")
    if algo == "returns":
        args = (nt, N, T, rp, te, tr, f64("trunc_values", (N, T)), f64("bootstrap", (N,)),
                gamma, out())
    elif algo in ("gae", "td_lambda"):
        args = (nt, N, T, rp, f64("values", (N, T + 1)), te, tr, f64("trunc_values", (N, T)),
                gamma, lam, out()) + ((out(),) if algo == "gae" else ())
    elif algo == "vtrace":
        args = (nt, N, T, rp, f64("values", (N, T + 1)), f64("log_rhos", (N, T)), te, tr,
                f64("trunc_values", (N, T)), gamma, lam, *clips, out(), out())
    elif algo == "retrace":
        args = (nt, N, T, rp, f64("q_taken", (N, T)), f64("exp_q_next", (N, T)),
                f64("log_rhos", (N, T)), te, tr, gamma, lam, clips[1], out())
    elif algo in ("eligibility_trace", "episodic_cumsum"):
        x = f64("bootstrap", (N,))
        args = (nt, N, T, rp, te, tr, x) + ((gamma, lam) if algo == "eligibility_trace"
                                             else ()) + (out(),)
    elif algo in ("retrace_probs", "vtrace_probs"):
        A = np.shape(_as_numpy(g("log_pi")))[2]
        S = T + 1 if algo == "retrace_probs" else T
        ac, acp = _i32(g("actions"), (N, T))
        keep.append(ac)
        mu_taken = len(np.shape(_as_numpy(g("log_mu")))) == 2
        lm = f64("log_mu", (N, T) if mu_taken else (N, T, A))
        if algo == "retrace_probs":
            args = (nt, N, T, A, rp, f64("q_values", (N, S, A)), acp, f64("log_pi", (N, S, A)),
                    lm, int(mu_taken), te, tr, f64("trunc_eq", (N, T)), gamma, lam, clips[1],
                    out())
        else:
            args = (nt, N, T, A, rp, f64("values", (N, T + 1)), acp, f64("log_pi", (N, S, A)),
                    lm, int(mu_taken), te, tr, f64("trunc_values", (N, T)), gamma, lam, *clips,
                    out(), out())
    else:
        raise ValueError("unknown algorithm %r" % (algo,))
    fn = getattr(lib, "oracle_rows_" + algo)

    def run():
        _check(fn(*args), algo + " (rows)")
        return outs

    run.inputs = keep
    return run
