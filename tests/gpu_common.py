"""Shared helpers for the GPU parity tests: run the HIP library and the oracle
on the same host inputs and compare.  Tolerances follow the stated bar:
max|gpu - ref| <= 1e-4 * max|ref| for fp32 inputs, 1e-2 * max|ref| for bf16
inputs (fp32 arithmetic in both cases)."""
import numpy as np
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from reverse_linear_recurrence_amd.synth import fp32_param

TOL = {"f32": 1e-4, "bf16": 1e-2}

ALGOS = ("returns", "gae", "td_lambda", "vtrace", "retrace", "eligibility", "cumsum")
FORWARD = ("eligibility", "cumsum")

DEFAULT_PARAMS = dict(gamma=0.97, lam=0.9, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0)


def params32(p):
    return {k: fp32_param(v) for k, v in p.items()}


def to_device(d, device="cuda"):
    return {k: v.to(device) for k, v in d.items()}


def run_gpu(algo, d, p, **kw):
    """Run one library call on device tensors d; returns dict name -> CPU float64 numpy."""
    g = lambda k: d.get(k)
    if algo == "returns":
        out = rl.rlca_returns(g("rewards"), g("terminated"), g("truncated"), g("trunc_values"),
                              g("bootstrap"), gamma=p["gamma"], **kw)
        res = {"returns": out}
    elif algo == "gae":
        adv, tgt = rl.rlca_gae(g("rewards"), g("values"), g("terminated"), g("truncated"),
                               g("trunc_values"), gamma=p["gamma"], lam=p["lam"], **kw)
        res = {"advantages": adv, "targets": tgt}
    elif algo == "td_lambda":
        res = {"lambda_returns": rl.rlca_td_lambda(g("rewards"), g("values"), g("terminated"),
                                                   g("truncated"), g("trunc_values"),
                                                   gamma=p["gamma"], lam=p["lam"], **kw)}
    elif algo == "vtrace":
        vs, pg = rl.rlca_vtrace(g("rewards"), g("values"), g("log_rhos"), g("terminated"),
                                g("truncated"), g("trunc_values"), gamma=p["gamma"], lam=p["lam"],
                                rho_bar=p["rho_bar"], c_bar=p["c_bar"],
                                pg_rho_bar=p["pg_rho_bar"], **kw)
        res = {"vs": vs, "pg_advantages": pg}
    elif algo == "retrace":
        res = {"q_ret": rl.rlca_retrace(g("rewards"), g("q_taken"), g("exp_q_next"),
                                        g("log_rhos"), g("terminated"), g("truncated"),
                                        gamma=p["gamma"], lam=p["lam"], c_bar=p["c_bar"], **kw)}
    elif algo == "eligibility":
        res = {"traces": rl.rlca_eligibility_trace(g("rewards"), g("terminated"), g("truncated"),
                                                   g("bootstrap"), gamma=p["gamma"],
                                                   lam=p["lam"], **kw)}
    elif algo == "cumsum":
        res = {"sums": rl.rlca_episodic_cumsum(g("rewards"), g("terminated"), g("truncated"),
                                               g("bootstrap"), **kw)}
    else:
        raise ValueError(algo)
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in res.items() if v is not None}


def run_oracle(algo, d, p):
    """The oracle on host copies of the same inputs (bf16 widened exactly)."""
    g = lambda k: None if d.get(k) is None else d[k].cpu()
    if algo == "returns":
        return {"returns": oracle.returns(g("rewards"), g("terminated"), g("truncated"),
                                          g("trunc_values"), g("bootstrap"), gamma=p["gamma"])}
    if algo == "gae":
        adv, tgt = oracle.gae(g("rewards"), g("values"), g("terminated"), g("truncated"),
                              g("trunc_values"), gamma=p["gamma"], lam=p["lam"])
        return {"advantages": adv, "targets": tgt}
    if algo == "td_lambda":
        return {"lambda_returns": oracle.td_lambda(g("rewards"), g("values"), g("terminated"),
                                                   g("truncated"), g("trunc_values"),
                                                   gamma=p["gamma"], lam=p["lam"])}
    if algo == "vtrace":
        vs, pg = oracle.vtrace(g("rewards"), g("values"), g("log_rhos"), g("terminated"),
                               g("truncated"), g("trunc_values"), gamma=p["gamma"], lam=p["lam"],
                               rho_bar=p["rho_bar"], c_bar=p["c_bar"], pg_rho_bar=p["pg_rho_bar"])
        return {"vs": vs, "pg_advantages": pg}
    if algo == "retrace":
        return {"q_ret": oracle.retrace(g("rewards"), g("q_taken"), g("exp_q_next"), g("log_rhos"),
                                        g("terminated"), g("truncated"), gamma=p["gamma"],
                                        lam=p["lam"], c_bar=p["c_bar"])}
    if algo == "eligibility":
        return {"traces": oracle.eligibility_trace(g("rewards"), g("terminated"), g("truncated"),
                                                   g("bootstrap"), gamma=p["gamma"],
                                                   lam=p["lam"])}
    if algo == "cumsum":
        return {"sums": oracle.episodic_cumsum(g("rewards"), g("terminated"), g("truncated"),
                                               g("bootstrap"))}
    raise ValueError(algo)


def rel_err(got, ref):
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(got - ref)))
    if scale == 0.0:
        return diff
    return diff / scale


def assert_close(got, ref, tol, what):
    for k in ref:
        assert k in got, "%s: missing output %s" % (what, k)
        assert got[k].shape == ref[k].shape, "%s/%s: shape %s vs %s" % (what, k, got[k].shape,
                                                                        ref[k].shape)
        assert np.all(np.isfinite(got[k])), "%s/%s: non-finite output" % (what, k)
        e = rel_err(got[k], ref[k])
        assert e <= tol, "%s/%s: max|err|/max|ref| = %.3g > %.1g" % (what, k, e, tol)


def random_inputs(algo, N, T, seed, dtype="f32", p_term=0.05, p_trunc=0.05, bootstrap=True):
    """Random inputs with dense boundaries (more than the benchmark's) to
    exercise every boundary path."""
    from reverse_linear_recurrence_amd.synth import make_rollout
    d = make_rollout(algo, N, T, seed=seed, dtype=dtype, p_term=p_term,
                     p_trunc=None if algo == "retrace" else p_trunc)
    if algo == "retrace" and p_trunc:
        g = np.random.Generator(np.random.PCG64(seed + 7))
        d["truncated"] = torch.from_numpy((g.random((N, T)) < p_trunc).astype(np.uint8))
    if algo in ("returns",) + FORWARD and bootstrap:
        g = np.random.Generator(np.random.PCG64(seed + 11))
        b = torch.from_numpy(g.standard_normal(N).astype(np.float32))
        d["bootstrap"] = b.to(torch.bfloat16) if dtype == "bf16" else b
    return d
