"""ctypes binding of librlca.so: argument marshalling only.

Each function mirrors the C entry point of the same name (include/rlca.h).
Tensors must be 2-D CUDA (HIP) tensors, contiguous along T (any row stride),
all floating-point inputs of one call share a dtype (float32 or bfloat16),
flags are bool or uint8.  Outputs are float32; they are allocated here unless
given.  The kernel is enqueued on ``stream`` (default: torch's current stream
of the tensors' device) and the call returns without synchronizing.
"""
import ctypes
import os

import torch

RLCA_OK, RLCA_EINVAL, RLCA_EDTYPE, RLCA_EALIAS, RLCA_EHIP = 0, 1, 2, 3, 4
RLCA_F32, RLCA_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librlca.so")
# The instrumented build (per-wavefront wall-clock stamps; see rlca_timestamps).
TIMED_LIB_PATH = os.path.join(_HERE, "librlca_timed.so")
# Loaded builds by path; calls go to the current one (librlca.so unless
# inside use_library).
_libs = {}
_current = _LIB_PATH

_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_vp = ctypes.c_void_p

_SIGNATURES = {
    "rlca_returns": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                     _f32, _vp, _i64, _vp],
    "rlca_gae": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                 _f32, _f32, _vp, _i64, _vp, _i64, _vp],
    "rlca_td_lambda": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                       _i64, _f32, _f32, _vp, _i64, _vp],
    "rlca_vtrace": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                    _vp, _i64, _f32, _f32, _f32, _f32, _f32, _vp, _i64, _vp, _i64, _vp],
    "rlca_retrace": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                     _vp, _i64, _f32, _f32, _f32, _vp, _i64, _vp],
    "rlca_eligibility_trace": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _f32,
                               _f32, _vp, _i64, _vp],
    "rlca_episodic_cumsum": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64,
                             _vp],
    "rlca_returns_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                           _f32, _vp, _i64, _vp, _vp, _vp, _i64, _vp],
    "rlca_gae_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                       _f32, _f32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp],
    "rlca_gae_chunk_noalloc": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                               _vp, _i64, _f32, _f32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp],
    "rlca_td_lambda_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                             _i64, _f32, _f32, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp],
    "rlca_vtrace_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                          _i64, _vp, _i64, _f32, _f32, _f32, _f32, _f32, _vp, _i64, _vp, _i64,
                          _vp, _vp, _vp, _vp, _i64, _vp],
    "rlca_retrace_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                           _i64, _vp, _i64, _f32, _f32, _f32, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp],
    "rlca_eligibility_trace_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                     _f32, _f32, _vp, _i64, _vp, _vp, _vp, _i64, _vp],
    "rlca_episodic_cumsum_chunk": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp,
                                   _i64, _vp, _vp, _vp, _i64, _vp],
    "rlca_affine_scan": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _int, _vp, _vp, _i64,
                         _vp, _vp, _vp, _i64, _vp],
    "rlca_retrace_probs": [_i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                           _vp, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _f32, _f32, _f32,
                           _vp, _i64, _vp],
    "rlca_vtrace_probs": [_i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                          _vp, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _f32, _f32, _f32,
                          _f32, _f32, _vp, _i64, _vp, _i64, _vp],
    "rlca_retrace_probs_chunk": [_i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                 _i64, _vp, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _f32,
                                 _f32, _f32, _vp, _i64, _vp, _vp, _vp, _vp],
    "rlca_vtrace_probs_chunk": [_i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                _i64, _vp, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _f32,
                                _f32, _f32, _f32, _f32, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                _vp],
    "rlca_materialized_workspace_bytes": [_i64, _i64],
    "rlca_returns_materialized": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                  _vp, _f32, _vp, _i64, _vp, _i64, _vp],
    "rlca_gae_materialized": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                              _i64, _f32, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _vp],
    "rlca_td_lambda_materialized": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                    _vp, _i64, _f32, _f32, _vp, _i64, _vp, _i64, _vp],
    "rlca_vtrace_materialized": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                 _vp, _i64, _vp, _i64, _f32, _f32, _f32, _f32, _f32, _vp, _i64,
                                 _vp, _i64, _vp, _i64, _vp],
    "rlca_retrace_materialized": [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                  _vp, _i64, _vp, _i64, _f32, _f32, _f32, _vp, _i64, _vp, _i64,
                                  _vp],
    "rlca_last_error": [],
    "rlca_version": [],
    "rlca_split_segments": [_i64, _i64],
    "rlca_split_workspace_bytes": [_i64, _i64],
    "rlca_timestamps": [_vp, _i64, ctypes.POINTER(_i64)],
    "rlca_num_variants": [],
    "rlca_set_variant": [_int],
    "rlca_variant_info": [_int, _int, _int, ctypes.POINTER(_int), ctypes.POINTER(_int),
                          ctypes.POINTER(_int)],
    "rlca_last_variant": [],
    "rlca_set_chained": [_int],
    "rlca_last_launches": [],
    "rlca_last_segments": [],
}


class RlcaError(RuntimeError):
    """A non-OK status from librlca; ``status`` holds the rlca_status code."""

    def __init__(self, status, message):
        super().__init__("rlca status %d: %s" % (status, message))
        self.status = status


def lib_path():
    return _LIB_PATH


def load_library(path=None):
    """Load librlca.so from the package directory (raises if it is not built)
    and return it; with ``path``, that build of the same ABI instead
    (TIMED_LIB_PATH: the instrumented one), without making it current (see
    use_library)."""
    path = path or _current
    lib = _libs.get(path)
    if lib is None:
        if not os.path.exists(path):
            raise ImportError("%s is not built: run `python -m reverse_linear_recurrence_amd.build"
                              "%s`" % (os.path.basename(path),
                                       " --timestamps" if path == TIMED_LIB_PATH else ""))
        lib = ctypes.CDLL(path)
        for name, argtypes in _SIGNATURES.items():
            if path != _LIB_PATH and not hasattr(lib, name):
                continue  # another build may predate an entry point
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = {"rlca_last_error": ctypes.c_char_p,
                          "rlca_split_workspace_bytes": ctypes.c_int64,
                          "rlca_materialized_workspace_bytes": ctypes.c_int64}.get(name,
                                                                                    ctypes.c_int)
        _libs[path] = lib
    return lib


class use_library:
    """``with use_library(path):`` routes this module's calls to another
    build of the library (e.g. TIMED_LIB_PATH) on the calling thread's
    behalf, for the duration of the block (not thread-safe: one current
    build per process)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _current
        load_library(self.path)
        self.prev, _current = _current, self.path
        return _libs[self.path]

    def __exit__(self, *exc):
        global _current
        _current = self.prev
        return False


def _check(rc):
    if rc != RLCA_OK:
        raise RlcaError(rc, load_library().rlca_last_error().decode())


def _float_input(name, x, dtype, shape, device):
    if x is None:
        return None, 0
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype != dtype:
        raise TypeError("%s has dtype %s; every float input of a call must be %s"
                        % (name, x.dtype, dtype))
    return _layout(name, x, shape, device)


def _flag_input(name, x, shape, device):
    if x is None:
        return None, 0
    if x.dtype not in (torch.bool, torch.uint8):
        raise TypeError("%s must be bool or uint8, got %s" % (name, x.dtype))
    return _layout(name, x, shape, device)


def _layout(name, x, shape, device):
    if x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    if len(shape) == 2:
        if shape[1] > 1 and x.stride(1) != 1:
            raise ValueError("%s must be contiguous along T (stride(1) == 1)" % name)
        ld = x.stride(0) if shape[0] > 1 else max(shape[1], 1)
        return x.data_ptr(), ld
    if shape[0] > 1 and x.stride(0) != 1:
        raise ValueError("%s must be contiguous" % name)
    return x.data_ptr(), 1


def _output(name, x, shape, device):
    if x is None:
        x = torch.empty(shape, dtype=torch.float32, device=device)
    elif x.dtype != torch.float32:
        raise TypeError("%s must be float32" % name)
    ptr, ld = _layout(name, x, shape, device)
    return x, ptr, ld


def _common(rewards):
    if not isinstance(rewards, torch.Tensor) or rewards.dim() != 2:
        raise ValueError("inputs must be 2-D tensors [num_envs, T]")
    if rewards.device.type != "cuda":
        raise ValueError("inputs must be on a GPU (got %s)" % rewards.device)
    if rewards.dtype == torch.float32:
        code = RLCA_F32
    elif rewards.dtype == torch.bfloat16:
        code = RLCA_BF16
    else:
        raise TypeError("float inputs must be float32 or bfloat16, got %s" % rewards.dtype)
    N, T = rewards.shape
    return N, T, code, rewards.device


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def rlca_returns(rewards, terminated=None, truncated=None, trunc_values=None, bootstrap=None,
                 *, gamma, out=None, stream=None):
    """Discounted returns [N, T] (float32).  bootstrap [N] is the carry G_T."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    b, _ = _float_input("bootstrap", bootstrap, dt, (N,), dev)
    out, o, ld_o = _output("returns", out, (N, T), dev)
    _check(load_library().rlca_returns(N, T, code, r, ld_r, te, ld_te, tr, ld_tr, tv, ld_tv, b,
                                       gamma, o, ld_o, _stream(stream, dev)))
    return out


def rlca_gae(rewards, values, terminated=None, truncated=None, trunc_values=None, *, gamma, lam,
             advantages=None, targets=None, with_targets=True, stream=None):
    """GAE advantages and value targets, each [N, T] float32.

    values is [N, T+1] (column T is the window bootstrap).  Returns
    ``(advantages, targets)``; targets is None when ``with_targets`` is False.
    """
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    adv, a, ld_a = _output("advantages", advantages, (N, T), dev)
    g, ld_g = None, 0
    if with_targets or targets is not None:
        targets, g, ld_g = _output("targets", targets, (N, T), dev)
    _check(load_library().rlca_gae(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr, ld_tr, tv, ld_tv,
                                   gamma, lam, a, ld_a, g, ld_g, _stream(stream, dev)))
    return adv, targets


def rlca_td_lambda(rewards, values, terminated=None, truncated=None, trunc_values=None, *, gamma,
                   lam, out=None, stream=None):
    """TD(lambda) returns [N, T] float32; values is [N, T+1]."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    out, o, ld_o = _output("lambda_returns", out, (N, T), dev)
    _check(load_library().rlca_td_lambda(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr, ld_tr, tv,
                                         ld_tv, gamma, lam, o, ld_o, _stream(stream, dev)))
    return out


def rlca_vtrace(rewards, values, log_rhos, terminated=None, truncated=None, trunc_values=None, *,
                gamma, lam=1.0, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0, vs=None,
                pg_advantages=None, with_pg=True, stream=None):
    """V-trace targets vs and policy-gradient advantages, each [N, T] float32.

    Returns ``(vs, pg_advantages)``; pg_advantages is None when ``with_pg`` is
    False.
    """
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    vs, o, ld_o = _output("vs", vs, (N, T), dev)
    pg, ld_pg = None, 0
    if with_pg or pg_advantages is not None:
        pg_advantages, pg, ld_pg = _output("pg_advantages", pg_advantages, (N, T), dev)
    _check(load_library().rlca_vtrace(N, T, code, r, ld_r, v, ld_v, lr, ld_lr, te, ld_te, tr,
                                      ld_tr, tv, ld_tv, gamma, lam, rho_bar, c_bar, pg_rho_bar,
                                      o, ld_o, pg, ld_pg, _stream(stream, dev)))
    return vs, pg_advantages


def rlca_retrace(rewards, q_taken, exp_q_next, log_rhos, terminated=None, truncated=None, *,
                 gamma, lam=1.0, c_bar=1.0, out=None, stream=None):
    """Retrace(lambda) targets Q^ret [N, T] float32."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    q, ld_q = _float_input("q_taken", q_taken, dt, (N, T), dev)
    eq, ld_eq = _float_input("exp_q_next", exp_q_next, dt, (N, T), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    out, o, ld_o = _output("q_ret", out, (N, T), dev)
    _check(load_library().rlca_retrace(N, T, code, r, ld_r, q, ld_q, eq, ld_eq, lr, ld_lr, te,
                                       ld_te, tr, ld_tr, gamma, lam, c_bar, o, ld_o,
                                       _stream(stream, dev)))
    return out


def rlca_eligibility_trace(x, terminated=None, truncated=None, z_init=None, *, gamma, lam,
                           out=None, stream=None):
    """Forward accumulating trace [N, T] float32:
    z_t = x_t + gamma*lam*(1-done_{t-1}) z_{t-1}, z_{-1} = z_init [N] (None: 0)."""
    N, T, code, dev = _common(x)
    dt = x.dtype
    a, ld_a = _float_input("x", x, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    z0, _ = _float_input("z_init", z_init, dt, (N,), dev)
    out, o, ld_o = _output("traces", out, (N, T), dev)
    _check(load_library().rlca_eligibility_trace(N, T, code, a, ld_a, te, ld_te, tr, ld_tr, z0,
                                                 gamma, lam, o, ld_o, _stream(stream, dev)))
    return out


def rlca_episodic_cumsum(x, terminated=None, truncated=None, s_init=None, *, out=None,
                         stream=None):
    """Forward episodic prefix sum [N, T] float32:
    S_t = x_t + (1-done_{t-1}) S_{t-1}, S_{-1} = s_init [N] (None: 0)."""
    N, T, code, dev = _common(x)
    dt = x.dtype
    a, ld_a = _float_input("x", x, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    s0, _ = _float_input("s_init", s_init, dt, (N,), dev)
    out, o, ld_o = _output("sums", out, (N, T), dev)
    _check(load_library().rlca_episodic_cumsum(N, T, code, a, ld_a, te, ld_te, tr, ld_tr, s0, o,
                                               ld_o, _stream(stream, dev)))
    return out


# ------------------------------------------------ materialized doubling scan
#
# rlca_X_materialized: the results of rlca_X through the materialized O(log T)
# doubling scan (the pages' comparison baseline, re-created in HIP), with a
# workspace of rlca_materialized_workspace_bytes(N, T) bytes (allocated here
# when not given).


def rlca_materialized_workspace_bytes(num_envs, T):
    b = load_library().rlca_materialized_workspace_bytes(int(num_envs), int(T))
    if b < 0:
        raise ValueError(load_library().rlca_last_error().decode())
    return b


def _mat_workspace(workspace, N, T, device):
    if workspace is None:
        workspace = torch.empty(rlca_materialized_workspace_bytes(N, T) // 4, dtype=torch.float32,
                                device=device)
    return (workspace,) + _workspace(workspace, device)


def rlca_returns_materialized(rewards, terminated=None, truncated=None, trunc_values=None,
                              bootstrap=None, *, gamma, out=None, workspace=None, stream=None):
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    b, _ = _float_input("bootstrap", bootstrap, dt, (N,), dev)
    out, o, ld_o = _output("returns", out, (N, T), dev)
    ws_t, ws, ws_b = _mat_workspace(workspace, N, T, dev)
    _check(load_library().rlca_returns_materialized(N, T, code, r, ld_r, te, ld_te, tr, ld_tr,
                                                    tv, ld_tv, b, gamma, o, ld_o, ws, ws_b,
                                                    _stream(stream, dev)))
    return out


def rlca_gae_materialized(rewards, values, terminated=None, truncated=None, trunc_values=None,
                          *, gamma, lam, advantages=None, targets=None, with_targets=True,
                          workspace=None, stream=None):
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    adv, a, ld_a = _output("advantages", advantages, (N, T), dev)
    g, ld_g = None, 0
    if with_targets or targets is not None:
        targets, g, ld_g = _output("targets", targets, (N, T), dev)
    ws_t, ws, ws_b = _mat_workspace(workspace, N, T, dev)
    _check(load_library().rlca_gae_materialized(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr,
                                                ld_tr, tv, ld_tv, gamma, lam, a, ld_a, g, ld_g,
                                                ws, ws_b, _stream(stream, dev)))
    return adv, targets


def rlca_td_lambda_materialized(rewards, values, terminated=None, truncated=None,
                                trunc_values=None, *, gamma, lam, out=None, workspace=None,
                                stream=None):
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    out, o, ld_o = _output("lambda_returns", out, (N, T), dev)
    ws_t, ws, ws_b = _mat_workspace(workspace, N, T, dev)
    _check(load_library().rlca_td_lambda_materialized(N, T, code, r, ld_r, v, ld_v, te, ld_te,
                                                      tr, ld_tr, tv, ld_tv, gamma, lam, o, ld_o,
                                                      ws, ws_b, _stream(stream, dev)))
    return out


def rlca_vtrace_materialized(rewards, values, log_rhos, terminated=None, truncated=None,
                             trunc_values=None, *, gamma, lam=1.0, rho_bar=1.0, c_bar=1.0,
                             pg_rho_bar=1.0, vs=None, pg_advantages=None, with_pg=True,
                             workspace=None, stream=None):
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    vs, o, ld_o = _output("vs", vs, (N, T), dev)
    pg, ld_pg = None, 0
    if with_pg or pg_advantages is not None:
        pg_advantages, pg, ld_pg = _output("pg_advantages", pg_advantages, (N, T), dev)
    ws_t, ws, ws_b = _mat_workspace(workspace, N, T, dev)
    _check(load_library().rlca_vtrace_materialized(N, T, code, r, ld_r, v, ld_v, lr, ld_lr, te,
                                                   ld_te, tr, ld_tr, tv, ld_tv, gamma, lam,
                                                   rho_bar, c_bar, pg_rho_bar, o, ld_o, pg,
                                                   ld_pg, ws, ws_b, _stream(stream, dev)))
    return vs, pg_advantages


def rlca_retrace_materialized(rewards, q_taken, exp_q_next, log_rhos, terminated=None,
                              truncated=None, *, gamma, lam=1.0, c_bar=1.0, out=None,
                              workspace=None, stream=None):
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    q, ld_q = _float_input("q_taken", q_taken, dt, (N, T), dev)
    eq, ld_eq = _float_input("exp_q_next", exp_q_next, dt, (N, T), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    out, o, ld_o = _output("q_ret", out, (N, T), dev)
    ws_t, ws, ws_b = _mat_workspace(workspace, N, T, dev)
    _check(load_library().rlca_retrace_materialized(N, T, code, r, ld_r, q, ld_q, eq, ld_eq, lr,
                                                    ld_lr, te, ld_te, tr, ld_tr, gamma, lam,
                                                    c_bar, o, ld_o, ws, ws_b,
                                                    _stream(stream, dev)))
    return out


# ------------------------------------------------------------ window calls
#
# Each rlca_X_chunk takes the arguments of rlca_X (the bootstrap / initial
# value replaced by ``carry_in``) and returns the outputs of rlca_X followed by
# ``carry_out`` [N] and ``carry_map`` [N, 2] (float32).  carry_in [N] float32
# (None: 0) is the scan state entering from the neighbouring window;
# carry_out must not overlap carry_in (use two vectors in turn).
# ``with_carry_out`` / ``with_map`` False pass NULL for that output (returned
# as None).  ``workspace`` (a contiguous GPU tensor, e.g. from
# split_workspace, or None) lets a call on few long rows run split.


def _workspace(workspace, device):
    if workspace is None:
        return None, 0
    if not (isinstance(workspace, torch.Tensor) and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    if workspace.device != device:
        raise ValueError("workspace is on %s, expected %s" % (workspace.device, device))
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _carry_in(carry_in, N, device):
    if carry_in is None:
        return None
    if not isinstance(carry_in, torch.Tensor) or carry_in.dtype != torch.float32:
        raise TypeError("carry_in must be a float32 tensor")
    ptr, _ = _layout("carry_in", carry_in, (N,), device)
    return ptr


def _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, device):
    co = cm = None
    co_p = cm_p = None
    if with_carry_out or carry_out is not None:
        carry_out, co_p, _ = _output("carry_out", carry_out, (N,), device)
        co = carry_out
    if with_map or carry_map is not None:
        if carry_map is None:
            carry_map = torch.empty((N, 2), dtype=torch.float32, device=device)
        if carry_map.dtype != torch.float32 or not carry_map.is_contiguous():
            raise TypeError("carry_map must be a contiguous float32 tensor")
        _layout("carry_map", carry_map, (N, 2), device)
        cm, cm_p = carry_map, carry_map.data_ptr()
    return co, cm, co_p, cm_p


def rlca_returns_chunk(rewards, terminated=None, truncated=None, trunc_values=None, *, gamma,
                       carry_in=None, out=None, carry_out=None, carry_map=None,
                       with_carry_out=True, with_map=True, workspace=None, stream=None):
    """Window of discounted returns: ``(returns, carry_out, carry_map)``;
    carry_in is G_T, carry_out is G_0."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("returns", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_returns_chunk(N, T, code, r, ld_r, te, ld_te, tr, ld_tr, tv, ld_tv,
                                             ci, gamma, o, ld_o, co_p, cm_p, ws, ws_b,
                                             _stream(stream, dev)))
    return out, co, cm


def rlca_gae_chunk(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
                   gamma, lam, carry_in=None, advantages=None, targets=None, with_targets=True,
                   carry_out=None, carry_map=None, with_carry_out=True, with_map=True,
                   workspace=None, stream=None):
    """Window of GAE: ``(advantages, targets, carry_out, carry_map)``; carry_in
    is the advantage A_T of the step after the window, carry_out is A_0."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    adv, a, ld_a = _output("advantages", advantages, (N, T), dev)
    g, ld_g = None, 0
    if with_targets or targets is not None:
        targets, g, ld_g = _output("targets", targets, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_gae_chunk(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr, ld_tr, tv,
                                         ld_tv, gamma, lam, a, ld_a, g, ld_g, ci, co_p, cm_p, ws,
                                         ws_b, _stream(stream, dev)))
    return adv, targets, co, cm


def rlca_gae_chunk_noalloc(rewards, values, terminated=None, truncated=None, trunc_values=None,
                           *, gamma, lam, carry_in=None, advantages=None, targets=None,
                           with_targets=True, carry_out=None, carry_map=None,
                           with_carry_out=True, with_map=True, stream=None):
    """rlca_gae_chunk for callers that cannot allocate: a call on few long
    rows splits with the library's own device scratch array instead of a
    workspace.  Pass every output (advantages, targets, carry_out, carry_map)
    to keep this wrapper from allocating them.  Calls that overlap in time on
    one device race on that array."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    adv, a, ld_a = _output("advantages", advantages, (N, T), dev)
    g, ld_g = None, 0
    if with_targets or targets is not None:
        targets, g, ld_g = _output("targets", targets, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    _check(load_library().rlca_gae_chunk_noalloc(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr,
                                                 ld_tr, tv, ld_tv, gamma, lam, a, ld_a, g, ld_g,
                                                 ci, co_p, cm_p, _stream(stream, dev)))
    return adv, targets, co, cm


def rlca_td_lambda_chunk(rewards, values, terminated=None, truncated=None, trunc_values=None, *,
                         gamma, lam, carry_in=None, out=None, carry_out=None, carry_map=None,
                         with_carry_out=True, with_map=True, workspace=None, stream=None):
    """Window of TD(lambda) returns: ``(lambda_returns, carry_out, carry_map)``;
    the carry is G^lambda - V (carry_in at step T, carry_out at step 0)."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("lambda_returns", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_td_lambda_chunk(N, T, code, r, ld_r, v, ld_v, te, ld_te, tr, ld_tr,
                                               tv, ld_tv, gamma, lam, o, ld_o, ci, co_p, cm_p, ws, ws_b,
                                               _stream(stream, dev)))
    return out, co, cm


def rlca_vtrace_chunk(rewards, values, log_rhos, terminated=None, truncated=None,
                      trunc_values=None, *, gamma, lam=1.0, rho_bar=1.0, c_bar=1.0,
                      pg_rho_bar=1.0, carry_in=None, vs=None, pg_advantages=None, with_pg=True,
                      carry_out=None, carry_map=None, with_carry_out=True, with_map=True,
                      workspace=None, stream=None):
    """Window of V-trace: ``(vs, pg_advantages, carry_out, carry_map)``; the
    carry is vs - V (carry_in at step T, carry_out at step 0)."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    vs, o, ld_o = _output("vs", vs, (N, T), dev)
    pg, ld_pg = None, 0
    if with_pg or pg_advantages is not None:
        pg_advantages, pg, ld_pg = _output("pg_advantages", pg_advantages, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_vtrace_chunk(N, T, code, r, ld_r, v, ld_v, lr, ld_lr, te, ld_te,
                                            tr, ld_tr, tv, ld_tv, gamma, lam, rho_bar, c_bar,
                                            pg_rho_bar, o, ld_o, pg, ld_pg, ci, co_p, cm_p, ws, ws_b,
                                            _stream(stream, dev)))
    return vs, pg_advantages, co, cm


def rlca_retrace_chunk(rewards, q_taken, exp_q_next, log_rhos, terminated=None, truncated=None,
                       *, gamma, lam=1.0, c_bar=1.0, carry_in=None, out=None, carry_out=None,
                       carry_map=None, with_carry_out=True, with_map=True, workspace=None,
                       stream=None):
    """Window of Retrace(lambda): ``(q_ret, carry_out, carry_map)``; the carry
    is c_t (q_ret_t - q_taken_t) (carry_in at step T, carry_out at step 0)."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    q, ld_q = _float_input("q_taken", q_taken, dt, (N, T), dev)
    eq, ld_eq = _float_input("exp_q_next", exp_q_next, dt, (N, T), dev)
    lr, ld_lr = _float_input("log_rhos", log_rhos, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("q_ret", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_retrace_chunk(N, T, code, r, ld_r, q, ld_q, eq, ld_eq, lr, ld_lr,
                                             te, ld_te, tr, ld_tr, gamma, lam, c_bar, o, ld_o, ci,
                                             co_p, cm_p, ws, ws_b, _stream(stream, dev)))
    return out, co, cm


def rlca_eligibility_trace_chunk(x, terminated=None, truncated=None, *, gamma, lam,
                                 carry_in=None, out=None, carry_out=None, carry_map=None,
                                 with_carry_out=True, with_map=True, workspace=None,
                                 stream=None):
    """Window of the eligibility trace: ``(traces, carry_out, carry_map)``;
    carry_in is z_{-1}, carry_out is z_{T-1} (0 if an episode ends there)."""
    N, T, code, dev = _common(x)
    dt = x.dtype
    a, ld_a = _float_input("x", x, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("traces", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_eligibility_trace_chunk(N, T, code, a, ld_a, te, ld_te, tr, ld_tr,
                                                       ci, gamma, lam, o, ld_o, co_p, cm_p, ws, ws_b,
                                                       _stream(stream, dev)))
    return out, co, cm


def rlca_episodic_cumsum_chunk(x, terminated=None, truncated=None, *, carry_in=None, out=None,
                               carry_out=None, carry_map=None, with_carry_out=True,
                               with_map=True, workspace=None, stream=None):
    """Window of the episodic prefix sum: ``(sums, carry_out, carry_map)``;
    carry_in is S_{-1}, carry_out is S_{T-1} (0 if an episode ends there)."""
    N, T, code, dev = _common(x)
    dt = x.dtype
    a, ld_a = _float_input("x", x, dt, (N, T), dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("sums", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_episodic_cumsum_chunk(N, T, code, a, ld_a, te, ld_te, tr, ld_tr,
                                                     ci, o, ld_o, co_p, cm_p, ws, ws_b,
                                                     _stream(stream, dev)))
    return out, co, cm


def rlca_affine_scan(alpha, beta, reset=None, *, reverse=True, carry_in=None, out=None,
                     carry_out=None, carry_map=None, with_carry_out=True, with_map=True,
                     workspace=None, stream=None):
    """Segmented affine scan: ``(A, carry_out, carry_map)`` with
    A_t = alpha_t + beta'_t A_{t+1} (reverse; A_T = carry_in) or
    A_t = alpha_t + beta'_t A_{t-1} (forward; A_{-1} = carry_in),
    beta'_t = 0 where reset_t, else beta_t."""
    N, T, code, dev = _common(alpha)
    dt = alpha.dtype
    a, ld_a = _float_input("alpha", alpha, dt, (N, T), dev)
    b, ld_b = _float_input("beta", beta, dt, (N, T), dev)
    rs, ld_rs = _flag_input("reset", reset, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("out", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    ws, ws_b = _workspace(workspace, dev)
    _check(load_library().rlca_affine_scan(N, T, code, a, ld_a, b, ld_b, rs, ld_rs,
                                           1 if reverse else 0, ci, o, ld_o, co_p, cm_p, ws, ws_b,
                                           _stream(stream, dev)))
    return out, co, cm


# ------------------------------------------------------ policy-table calls


def _table(name, x, dtype, N, S, A, device):
    """A [N, S, A] table, contiguous within a row: (pointer, row stride in elements)."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dtype != dtype:
        raise TypeError("%s has dtype %s; every float input of a call must be %s"
                        % (name, x.dtype, dtype))
    if x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if tuple(x.shape) != (N, S, A):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), (N, S, A)))
    if (A > 1 and x.stride(2) != 1) or (S > 1 and x.stride(1) != A):
        raise ValueError("%s must be contiguous within a row ([N, S, A] with strides (ld, A, 1))"
                         % name)
    ld = x.stride(0) if N > 1 else max(S * A, 1)
    return x.data_ptr(), ld


def _actions(x, N, T, device):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.int32:
        raise TypeError("actions must be an int32 tensor")
    return _layout("actions", x, (N, T), device)


def _log_mu(log_mu, dtype, N, T, A, device):
    """log_mu as a [N, T, A] table, or [N, T]: the taken actions' entries."""
    if isinstance(log_mu, torch.Tensor) and log_mu.dim() == 2:
        ptr, ld = _float_input("log_mu", log_mu, dtype, (N, T), device)
        return ptr, ld, 1
    ptr, ld = _table("log_mu", log_mu, dtype, N, T, A, device)
    return ptr, ld, 0


def rlca_retrace_probs(rewards, q_values, actions, log_pi, log_mu, terminated=None,
                       truncated=None, trunc_eq=None, *, gamma, lam=1.0, c_bar=1.0, out=None,
                       stream=None):
    """Retrace(lambda) targets [N, T] float32 from q_values and log_pi
    [N, T+1, A], log_mu [N, T, A] (or [N, T]: the taken actions' entries) and
    int32 actions [N, T]; trunc_eq [N, T] (E_pi Q at the true final state) is
    read at truncations."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    if not isinstance(q_values, torch.Tensor) or q_values.dim() != 3:
        raise ValueError("q_values must be a 3-D tensor [N, T+1, A]")
    A = q_values.shape[2]
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    q, ld_q = _table("q_values", q_values, dt, N, T + 1, A, dev)
    ac, ld_ac = _actions(actions, N, T, dev)
    lp, ld_lp = _table("log_pi", log_pi, dt, N, T + 1, A, dev)
    lm, ld_lm, mu_taken = _log_mu(log_mu, dt, N, T, A, dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    teq, ld_teq = _float_input("trunc_eq", trunc_eq, dt, (N, T), dev)
    out, o, ld_o = _output("q_ret", out, (N, T), dev)
    _check(load_library().rlca_retrace_probs(N, T, A, code, r, ld_r, q, ld_q, ac, ld_ac, lp, ld_lp,
                                             lm, ld_lm, mu_taken, te, ld_te, tr, ld_tr, teq,
                                             ld_teq, gamma, lam, c_bar, o, ld_o,
                                             _stream(stream, dev)))
    return out


def rlca_vtrace_probs(rewards, values, actions, log_pi, log_mu, terminated=None, truncated=None,
                      trunc_values=None, *, gamma, lam=1.0, rho_bar=1.0, c_bar=1.0,
                      pg_rho_bar=1.0, vs=None, pg_advantages=None, with_pg=True, stream=None):
    """V-trace from log_pi [N, T, A], log_mu [N, T, A] (or [N, T]: the taken
    actions' entries) and int32 actions [N, T]: ``(vs, pg_advantages)``,
    each [N, T] float32."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    if not isinstance(log_pi, torch.Tensor) or log_pi.dim() != 3:
        raise ValueError("log_pi must be a 3-D tensor [N, T, A]")
    A = log_pi.shape[2]
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    ac, ld_ac = _actions(actions, N, T, dev)
    lp, ld_lp = _table("log_pi", log_pi, dt, N, T, A, dev)
    lm, ld_lm, mu_taken = _log_mu(log_mu, dt, N, T, A, dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    vs, o, ld_o = _output("vs", vs, (N, T), dev)
    pg, ld_pg = None, 0
    if with_pg or pg_advantages is not None:
        pg_advantages, pg, ld_pg = _output("pg_advantages", pg_advantages, (N, T), dev)
    _check(load_library().rlca_vtrace_probs(N, T, A, code, r, ld_r, v, ld_v, ac, ld_ac, lp, ld_lp,
                                            lm, ld_lm, mu_taken, te, ld_te, tr, ld_tr, tv, ld_tv,
                                            gamma, lam, rho_bar, c_bar, pg_rho_bar, o, ld_o, pg,
                                            ld_pg, _stream(stream, dev)))
    return vs, pg_advantages


def rlca_retrace_probs_chunk(rewards, q_values, actions, log_pi, log_mu, terminated=None,
                             truncated=None, trunc_eq=None, *, gamma, lam=1.0, c_bar=1.0,
                             carry_in=None, out=None, carry_out=None, carry_map=None,
                             with_carry_out=True, with_map=True, stream=None):
    """Window of rlca_retrace_probs: ``(q_ret, carry_out, carry_map)``; the
    carry is c_t (q_ret_t - q_taken_t) (carry_in at step T, carry_out at 0)."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    if not isinstance(q_values, torch.Tensor) or q_values.dim() != 3:
        raise ValueError("q_values must be a 3-D tensor [N, T+1, A]")
    A = q_values.shape[2]
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    q, ld_q = _table("q_values", q_values, dt, N, T + 1, A, dev)
    ac, ld_ac = _actions(actions, N, T, dev)
    lp, ld_lp = _table("log_pi", log_pi, dt, N, T + 1, A, dev)
    lm, ld_lm, mu_taken = _log_mu(log_mu, dt, N, T, A, dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    teq, ld_teq = _float_input("trunc_eq", trunc_eq, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    out, o, ld_o = _output("q_ret", out, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    _check(load_library().rlca_retrace_probs_chunk(
        N, T, A, code, r, ld_r, q, ld_q, ac, ld_ac, lp, ld_lp, lm, ld_lm, mu_taken, te, ld_te,
        tr, ld_tr, teq, ld_teq, gamma, lam, c_bar, o, ld_o, ci, co_p, cm_p,
        _stream(stream, dev)))
    return out, co, cm


def rlca_vtrace_probs_chunk(rewards, values, actions, log_pi, log_mu, terminated=None,
                            truncated=None, trunc_values=None, *, gamma, lam=1.0, rho_bar=1.0,
                            c_bar=1.0, pg_rho_bar=1.0, carry_in=None, vs=None,
                            pg_advantages=None, with_pg=True, carry_out=None, carry_map=None,
                            with_carry_out=True, with_map=True, stream=None):
    """Window of rlca_vtrace_probs: ``(vs, pg_advantages, carry_out, carry_map)``;
    the carry is vs - V (carry_in at step T, carry_out at step 0)."""
    N, T, code, dev = _common(rewards)
    dt = rewards.dtype
    if not isinstance(log_pi, torch.Tensor) or log_pi.dim() != 3:
        raise ValueError("log_pi must be a 3-D tensor [N, T, A]")
    A = log_pi.shape[2]
    r, ld_r = _float_input("rewards", rewards, dt, (N, T), dev)
    v, ld_v = _float_input("values", values, dt, (N, T + 1), dev)
    ac, ld_ac = _actions(actions, N, T, dev)
    lp, ld_lp = _table("log_pi", log_pi, dt, N, T, A, dev)
    lm, ld_lm, mu_taken = _log_mu(log_mu, dt, N, T, A, dev)
    te, ld_te = _flag_input("terminated", terminated, (N, T), dev)
    tr, ld_tr = _flag_input("truncated", truncated, (N, T), dev)
    tv, ld_tv = _float_input("trunc_values", trunc_values, dt, (N, T), dev)
    ci = _carry_in(carry_in, N, dev)
    vs, o, ld_o = _output("vs", vs, (N, T), dev)
    pg, ld_pg = None, 0
    if with_pg or pg_advantages is not None:
        pg_advantages, pg, ld_pg = _output("pg_advantages", pg_advantages, (N, T), dev)
    co, cm, co_p, cm_p = _carry_outputs(carry_out, carry_map, with_carry_out, with_map, N, dev)
    _check(load_library().rlca_vtrace_probs_chunk(
        N, T, A, code, r, ld_r, v, ld_v, ac, ld_ac, lp, ld_lp, lm, ld_lm, mu_taken, te, ld_te,
        tr, ld_tr, tv, ld_tv, gamma, lam, rho_bar, c_bar, pg_rho_bar, o, ld_o, pg, ld_pg, ci,
        co_p, cm_p, _stream(stream, dev)))
    return vs, pg_advantages, co, cm


def rlca_version():
    return load_library().rlca_version()


def rlca_num_variants():
    return load_library().rlca_num_variants()


def rlca_set_variant(variant):
    """Force tiling variant ``variant`` on this thread (-1: automatic); returns the previous."""
    prev = load_library().rlca_set_variant(int(variant))
    if prev == -2:
        raise ValueError("unknown variant %r" % (variant,))
    return prev


# Algorithm codes of rlca_variant_info (rlca_algo); a window form takes its
# algorithm's code, the affine scan "affine" in either direction.
ALGO_CODES = {"returns": 0, "gae": 1, "td_lambda": 2, "vtrace": 3, "retrace": 4,
              "eligibility": 5, "cumsum": 6, "affine": 7}


def rlca_variant_info(variant, dtype=torch.float32, algo="gae"):
    """(steps_per_lane, lanes_per_row, waves_per_row) of a tiling variant for
    the algorithm ``algo`` (a key of ALGO_CODES) on inputs of ``dtype``
    (torch.float32 or torch.bfloat16)."""
    code = RLCA_BF16 if dtype in (torch.bfloat16, RLCA_BF16, "bf16") else RLCA_F32
    if algo not in ALGO_CODES:
        raise ValueError("unknown algorithm %r" % (algo,))
    k, l, w = _int(), _int(), _int()
    _check(load_library().rlca_variant_info(int(variant), ALGO_CODES[algo], code,
                                            ctypes.byref(k), ctypes.byref(l), ctypes.byref(w)))
    return k.value, l.value, w.value


def rlca_split_segments(num_envs, T):
    """Segments per row a window call of num_envs rows of T steps is split
    into when given a workspace (1: not split)."""
    s = load_library().rlca_split_segments(int(num_envs), int(T))
    if s < 0:
        raise ValueError(load_library().rlca_last_error().decode())
    return s


def rlca_split_workspace_bytes(num_envs, T):
    """Workspace bytes a split window call of num_envs rows of T steps needs
    (0: the call does not split)."""
    b = load_library().rlca_split_workspace_bytes(int(num_envs), int(T))
    if b < 0:
        raise ValueError(load_library().rlca_last_error().decode())
    return b


def split_workspace(num_envs, T, device="cuda"):
    """A workspace tensor for a window call of num_envs rows of T steps, or
    None when the call would not split."""
    b = rlca_split_workspace_bytes(num_envs, T)
    if b == 0:
        return None
    return torch.empty(b // 4, dtype=torch.float32, device=device)


def rlca_timestamps(max_waves=1 << 16):
    """Instrumented build only: the (start, end) wall-clock stamps, in ticks
    of 10 ns, of every wavefront of the calling thread's last launch, as a
    uint64 numpy array [waves, 2].  Synchronizes with the device."""
    import numpy as np
    buf = (ctypes.c_uint64 * (2 * max_waves))()
    n = _i64()
    _check(load_library().rlca_timestamps(ctypes.cast(buf, _vp), int(max_waves),
                                          ctypes.byref(n)))
    return np.frombuffer(buf, dtype=np.uint64, count=2 * n.value).reshape(-1, 2).copy()


def rlca_last_variant():
    return load_library().rlca_last_variant()


def rlca_set_chained(enable):
    """Allow (True, the default) or forbid the one-launch chained form of
    split calls on this thread; returns the previous setting."""
    return bool(load_library().rlca_set_chained(1 if enable else 0))


def rlca_last_launches():
    """Kernel launches the calling thread's last successful call enqueued."""
    return load_library().rlca_last_launches()


def rlca_last_segments():
    """Segments per row of the calling thread's last successful call (1: not split)."""
    return load_library().rlca_last_segments()
