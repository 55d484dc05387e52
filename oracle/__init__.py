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
"""
import ctypes
import os

import numpy as np

from .build import LIB, SRC, build_oracle

_lib = None
_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        i64, dbl = ctypes.c_int64, ctypes.c_double
        lib.oracle_returns.argtypes = [i64, i64, _D, _U8, _U8, _D, _D, dbl, _D]
        lib.oracle_gae.argtypes = [i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D, _D]
        lib.oracle_td_lambda.argtypes = [i64, i64, _D, _D, _U8, _U8, _D, dbl, dbl, _D]
        lib.oracle_vtrace.argtypes = [i64, i64, _D, _D, _D, _U8, _U8, _D,
                                      dbl, dbl, dbl, dbl, dbl, _D, _D]
        lib.oracle_retrace.argtypes = [i64, i64, _D, _D, _D, _D, _U8, _U8,
                                       dbl, dbl, dbl, _D]
        lib.oracle_eligibility_trace.argtypes = [i64, i64, _D, _U8, _U8, _D, dbl, dbl, _D]
        lib.oracle_episodic_cumsum.argtypes = [i64, i64, _D, _U8, _U8, _D, _D]
        for f in (lib.oracle_returns, lib.oracle_gae, lib.oracle_td_lambda,
                  lib.oracle_vtrace, lib.oracle_retrace, lib.oracle_eligibility_trace,
                  lib.oracle_episodic_cumsum):
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


def returns(rewards, terminated=None, truncated=None, trunc_values=None,
            bootstrap=None, *, gamma):
    """Discounted returns ``G [N, T]``; ``bootstrap [N]`` is the carry ``G_T`` (None: 0)."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    b, bp = _f64(bootstrap, (N,))
    out = np.empty((N, T), np.float64)
    _check(_load().oracle_returns(N, T, rp, tep, trp, tvp, bp, float(gamma),
                                  out.ctypes.data_as(_D)), "returns")
    return out


def gae(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
        gamma, lam):
    """GAE: returns ``(advantages, targets)``, each ``[N, T]``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    adv = np.empty((N, T), np.float64)
    tgt = np.empty((N, T), np.float64)
    _check(_load().oracle_gae(N, T, rp, vp, tep, trp, tvp, float(gamma), float(lam),
                              adv.ctypes.data_as(_D), tgt.ctypes.data_as(_D)), "gae")
    return adv, tgt


def td_lambda(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
              gamma, lam):
    """TD(lambda) returns ``[N, T]``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    out = np.empty((N, T), np.float64)
    _check(_load().oracle_td_lambda(N, T, rp, vp, tep, trp, tvp, float(gamma), float(lam),
                                    out.ctypes.data_as(_D)), "td_lambda")
    return out


def vtrace(rewards, values, log_rhos, terminated=None, truncated=None, trunc_values=None,
           *, gamma, lam, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0):
    """V-trace: returns ``(vs, pg_advantages)``, each ``[N, T]``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    v, vp = _f64(values, (N, T + 1))
    lr, lrp = _f64(log_rhos, (N, T))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    tv, tvp = _f64(trunc_values, (N, T))
    vs = np.empty((N, T), np.float64)
    pg = np.empty((N, T), np.float64)
    _check(_load().oracle_vtrace(N, T, rp, vp, lrp, tep, trp, tvp, float(gamma), float(lam),
                                 float(rho_bar), float(c_bar), float(pg_rho_bar),
                                 vs.ctypes.data_as(_D), pg.ctypes.data_as(_D)), "vtrace")
    return vs, pg


def retrace(rewards, q_taken, exp_q_next, log_rhos, terminated=None, truncated=None, *,
            gamma, lam, c_bar=1.0):
    """Retrace(lambda) targets ``Q^ret [N, T]``."""
    r, rp = _f64(rewards, np.shape(_as_numpy(rewards)))
    N, T = r.shape
    q, qp = _f64(q_taken, (N, T))
    eq, eqp = _f64(exp_q_next, (N, T))
    lr, lrp = _f64(log_rhos, (N, T))
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    out = np.empty((N, T), np.float64)
    _check(_load().oracle_retrace(N, T, rp, qp, eqp, lrp, tep, trp, float(gamma), float(lam),
                                  float(c_bar), out.ctypes.data_as(_D)), "retrace")
    return out


def eligibility_trace(x, terminated=None, truncated=None, z_init=None, *, gamma, lam):
    """Forward accumulating trace ``z [N, T]``: z_t = x_t + gamma*lam*(1-done_{t-1}) z_{t-1}."""
    a, ap = _f64(x, np.shape(_as_numpy(x)))
    N, T = a.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    z0, z0p = _f64(z_init, (N,))
    out = np.empty((N, T), np.float64)
    _check(_load().oracle_eligibility_trace(N, T, ap, tep, trp, z0p, float(gamma), float(lam),
                                            out.ctypes.data_as(_D)), "eligibility_trace")
    return out


def episodic_cumsum(x, terminated=None, truncated=None, s_init=None):
    """Forward episodic prefix sum ``S [N, T]``: S_t = x_t + (1-done_{t-1}) S_{t-1}."""
    a, ap = _f64(x, np.shape(_as_numpy(x)))
    N, T = a.shape
    te, tep = _u8(terminated, (N, T))
    tr, trp = _u8(truncated, (N, T))
    s0, s0p = _f64(s_init, (N,))
    out = np.empty((N, T), np.float64)
    _check(_load().oracle_episodic_cumsum(N, T, ap, tep, trp, s0p, out.ctypes.data_as(_D)),
           "episodic_cumsum")
    return out
