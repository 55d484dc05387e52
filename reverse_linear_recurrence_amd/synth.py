"""Seeded synthetic rollouts for the credit-assignment workloads.

This module only draws random inputs; it holds none of the method's
arithmetic.  The test suite and the benchmark feed the same draws to the HIP
library and to the CPU oracle.

Draws use ``numpy.random.Generator(PCG64(seed))`` in a fixed order:
rewards, values, q_taken, exp_q_next, log_rhos, terminated, truncated,
trunc_values.  An array that a workload does not use is not drawn, so the
order of the draws that remain is unchanged.  Bernoulli flags are ``u < p``
stored as ``uint8``.  bf16 inputs are rounded from the fp32 draws by torch
(round-to-nearest-even) on the CPU, so both sides see identical bits.

Workloads follow the synthetic rollout shapes the rl-triton explainer pages
discuss (``[num_envs, seq_len]`` tensors, Technical summary: Problem; results
quoted at 4096 envs x 128 steps).  The five named workloads below are the
configurations this library is measured on; the policy-table workloads draw
their tables with ``make_tables``.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    algo: str                 # returns | gae | td_lambda | vtrace | retrace | vtrace+retrace
    num_envs: int
    T: int
    dtype: str                # "f32" | "bf16": dtype of every floating-point input
    seed: int
    gamma: float
    lam: float = 1.0
    p_term: float = 0.0
    p_trunc: Optional[float] = None   # None: no truncation array at all
    reward_dist: str = "normal"       # "normal" N(0,1) | "uniform" U(-1,1)
    log_rho_std: float = 0.5
    clips: Dict[str, float] = field(default_factory=dict)
    num_actions: int = 0              # policy-table workloads: actions per step
    mu_taken: bool = False            # log_mu as the taken actions' entries [N, T]


WORKLOADS = {
    "returns_4x128": Workload("returns_4x128", "returns", 4, 128, "f32", 101,
                              gamma=0.99, p_term=0.01),
    "gae_4096x128": Workload("gae_4096x128", "gae", 4096, 128, "f32", 102,
                             gamma=0.99, lam=0.95, p_term=0.005, p_trunc=0.002),
    "td_lambda_16384x256": Workload("td_lambda_16384x256", "td_lambda", 16384, 256, "f32",
                                    103, gamma=0.995, lam=0.9, p_term=0.004,
                                    reward_dist="uniform"),
    "offpolicy_2048x1024": Workload("offpolicy_2048x1024", "vtrace+retrace", 2048, 1024,
                                    "f32", 104, gamma=0.99, lam=0.95, p_term=0.002,
                                    clips={"rho_bar": 1.0, "c_bar": 1.0, "pg_rho_bar": 1.0}),
    "gae_bf16_256x16384": Workload("gae_bf16_256x16384", "gae", 256, 16384, "bf16", 105,
                                   gamma=0.999, lam=0.97, p_term=0.0005, p_trunc=0.0002),
    # Few long rows (split calls when a workspace is set), at the long-horizon
    # workload's rates.
    "gae_bf16_16x262144": Workload("gae_bf16_16x262144", "gae", 16, 262144, "bf16", 110,
                                   gamma=0.999, lam=0.97, p_term=0.0005, p_trunc=0.0002),
    # Fewer rows than CUs but more than a few: 160 rows leave 96 CUs idle
    # unsplit.
    "gae_bf16_160x32768": Workload("gae_bf16_160x32768", "gae", 160, 32768, "bf16", 111,
                                   gamma=0.999, lam=0.97, p_term=0.0005, p_trunc=0.0002),
    # Forward-time mirrors, at the GAE workload's shape and boundary rates.
    "eligibility_4096x128": Workload("eligibility_4096x128", "eligibility", 4096, 128, "f32",
                                     106, gamma=0.99, lam=0.95, p_term=0.005, p_trunc=0.002),
    "cumsum_4096x128": Workload("cumsum_4096x128", "cumsum", 4096, 128, "f32", 107,
                                gamma=1.0, lam=1.0, p_term=0.005, p_trunc=0.002),
    # Retrace and V-trace from policy tables, at the off-policy workload's
    # shape with 18 actions (the size of a full Atari action set).
    "retrace_probs_2048x1024x18": Workload("retrace_probs_2048x1024x18", "retrace_probs", 2048,
                                           1024, "f32", 108, gamma=0.99, lam=0.95,
                                           p_term=0.002, p_trunc=0.001,
                                           clips={"c_bar": 1.0}, num_actions=18,
                                           mu_taken=True),
    "vtrace_probs_2048x1024x18": Workload("vtrace_probs_2048x1024x18", "vtrace_probs", 2048,
                                          1024, "f32", 109, gamma=0.99, lam=0.95,
                                          p_term=0.002, p_trunc=0.001,
                                          clips={"rho_bar": 1.0, "c_bar": 1.0, "pg_rho_bar": 1.0},
                                          num_actions=18),
}

_NEEDS = {
    "returns": ("rewards",),
    "gae": ("rewards", "values"),
    "td_lambda": ("rewards", "values"),
    "vtrace": ("rewards", "values", "log_rhos"),
    "retrace": ("rewards", "q_taken", "exp_q_next", "log_rhos"),
    "vtrace+retrace": ("rewards", "values", "q_taken", "exp_q_next", "log_rhos"),
    # forward-time algorithms: the per-step input x is drawn as "rewards"
    "eligibility": ("rewards",),
    "cumsum": ("rewards",),
}
_FORWARD = ("eligibility", "cumsum")


def fp32_param(x: float) -> float:
    """The float32 value of a scalar parameter, widened back to a Python float.

    The library takes gamma, lambda and the clips as float32; the oracle is fed
    the same rounded values.
    """
    return float(np.float32(x))


def make_rollout(algo: str, num_envs: int, T: int, *, seed: int, dtype: str = "f32",
                 p_term: float = 0.0, p_trunc: Optional[float] = None,
                 reward_dist: str = "normal", log_rho_std: float = 0.5,
                 dense_trunc_values: bool = True) -> Dict[str, torch.Tensor]:
    """Draw one rollout batch as CPU tensors.

    Returns a dict with (as the algorithm needs) ``rewards [N,T]``,
    ``values [N,T+1]``, ``q_taken [N,T]``, ``exp_q_next [N,T]``,
    ``log_rhos [N,T]``, ``terminated [N,T] uint8``, ``truncated [N,T] uint8``
    (only if ``p_trunc`` is not None) and ``trunc_values [N,T]`` (with
    truncations, drawn densely: entries that are not truncation bootstraps are
    never read by a correct implementation, so they hold live random values).
    """
    if algo not in _NEEDS:
        raise ValueError("unknown algorithm %r" % algo)
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    g = np.random.Generator(np.random.PCG64(seed))
    N = num_envs
    need = _NEEDS[algo]
    out: Dict[str, np.ndarray] = {}
    if reward_dist == "normal":
        out["rewards"] = g.standard_normal((N, T), dtype=np.float32)
    elif reward_dist == "uniform":
        out["rewards"] = g.uniform(-1.0, 1.0, (N, T)).astype(np.float32)
    else:
        raise ValueError("reward_dist must be 'normal' or 'uniform'")
    if "values" in need:
        out["values"] = g.standard_normal((N, T + 1), dtype=np.float32)
    if "q_taken" in need:
        out["q_taken"] = g.standard_normal((N, T), dtype=np.float32)
        out["exp_q_next"] = g.standard_normal((N, T), dtype=np.float32)
    if "log_rhos" in need:
        out["log_rhos"] = (g.standard_normal((N, T), dtype=np.float32)
                           * np.float32(log_rho_std)).astype(np.float32)
    out["terminated"] = (g.random((N, T)) < p_term).astype(np.uint8)
    if p_trunc is not None:
        out["truncated"] = (g.random((N, T)) < p_trunc).astype(np.uint8)
        if algo in _FORWARD:
            pass  # no bootstrap values: forward recurrences only restart
        elif dense_trunc_values:
            out["trunc_values"] = g.standard_normal((N, T), dtype=np.float32)
        else:
            out["trunc_values"] = np.zeros((N, T), np.float32)
    res: Dict[str, torch.Tensor] = {}
    for k, a in out.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bf16" and a.dtype == np.float32:
            t = t.to(torch.bfloat16)
        res[k] = t
    return res


def _log_probs(g: np.random.Generator, shape, scale: float) -> np.ndarray:
    """Log-probability tables of random policies: N(0, scale^2) logits,
    normalized over the last axis (in float64, then rounded to float32)."""
    z = g.standard_normal(shape) * scale
    z = z - z.max(-1, keepdims=True)
    return (z - np.log(np.exp(z).sum(-1, keepdims=True))).astype(np.float32)


def make_tables(algo: str, num_envs: int, T: int, num_actions: int, *, seed: int,
                dtype: str = "f32", p_term: float = 0.0, p_trunc: Optional[float] = None,
                logit_scale: float = 1.0, mu_taken: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one batch for the policy-table entry points as CPU tensors.

    Draw order: rewards [N,T]; values [N,T+1] (vtrace_probs) or q_values
    [N,T+1,A] (retrace_probs); target log-probabilities log_pi ([N,T+1,A]
    for Retrace, [N,T,A] for V-trace); behaviour log-probabilities log_mu
    [N,T,A]; actions [N,T] int32, sampled from the behaviour policy by
    inverse CDF of uniform draws; terminated; truncated (if p_trunc is not
    None) with trunc_eq (Retrace) or trunc_values (V-trace) [N,T], drawn
    densely as N(0,1).  mu_taken: log_mu is returned as the taken actions'
    entries [N,T] (the same draws).
    """
    if algo not in ("retrace_probs", "vtrace_probs"):
        raise ValueError("unknown policy-table algorithm %r" % algo)
    g = np.random.Generator(np.random.PCG64(seed))
    N, A = num_envs, num_actions
    retrace = algo == "retrace_probs"
    out: Dict[str, np.ndarray] = {"rewards": g.standard_normal((N, T), dtype=np.float32)}
    if retrace:
        out["q_values"] = g.standard_normal((N, T + 1, A), dtype=np.float32)
        out["log_pi"] = _log_probs(g, (N, T + 1, A), logit_scale)
    else:
        out["values"] = g.standard_normal((N, T + 1), dtype=np.float32)
        out["log_pi"] = _log_probs(g, (N, T, A), logit_scale)
    out["log_mu"] = _log_probs(g, (N, T, A), logit_scale)
    cdf = np.cumsum(np.exp(out["log_mu"].astype(np.float64)), axis=-1)
    u = g.random((N, T, 1)) * cdf[..., -1:]
    out["actions"] = np.minimum((cdf < u).sum(-1), A - 1).astype(np.int32)
    if mu_taken:
        out["log_mu"] = np.take_along_axis(out["log_mu"], out["actions"][..., None].astype(np.int64),
                                           -1)[..., 0]
    out["terminated"] = (g.random((N, T)) < p_term).astype(np.uint8)
    if p_trunc is not None:
        out["truncated"] = (g.random((N, T)) < p_trunc).astype(np.uint8)
        out["trunc_eq" if retrace else "trunc_values"] = g.standard_normal((N, T),
                                                                           dtype=np.float32)
    res: Dict[str, torch.Tensor] = {}
    for k, a in out.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bf16" and a.dtype == np.float32:
            t = t.to(torch.bfloat16)
        res[k] = t
    return res


def make_workload(w: Workload, num_envs: Optional[int] = None, T: Optional[int] = None,
                  seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of a named workload (optionally at another size or seed)."""
    if w.algo in ("retrace_probs", "vtrace_probs"):
        return make_tables(w.algo, num_envs or w.num_envs, T or w.T, w.num_actions,
                           seed=w.seed if seed is None else seed, dtype=w.dtype,
                           p_term=w.p_term, p_trunc=w.p_trunc, mu_taken=w.mu_taken)
    return make_rollout(w.algo, num_envs or w.num_envs, T or w.T,
                        seed=w.seed if seed is None else seed, dtype=w.dtype,
                        p_term=w.p_term, p_trunc=w.p_trunc, reward_dist=w.reward_dist,
                        log_rho_std=w.log_rho_std)
