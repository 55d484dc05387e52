"""GPU parity of the materialized doubling scan (rlca_X_materialized), the
comparison baseline of the rl-triton pages (Technical summary, Problem: a
vectorized O(log T) scan that materializes its intermediates in HBM)
re-created in HIP: (alpha, beta) of every step written out, ceil(log2 T)
doubling passes, then the outputs.  It must match the oracle at the same bar
as the fused entry points (max|err| <= 1e-4 max|ref| for fp32 inputs, 1e-2
for bf16 inputs): on random inputs with dense boundaries, at lengths around
the powers of two the passes double through, on strided rows, and on the
five benchmark configurations at full size."""
import numpy as np
import pytest
import torch

import oracle
import reverse_linear_recurrence_amd as rl
from gpu_common import (DEFAULT_PARAMS, TOL, assert_close, params32, random_inputs, run_gpu,
                        run_oracle, to_device)
from reverse_linear_recurrence_amd.synth import WORKLOADS, fp32_param, make_workload
from test_gpu_parity import EXTREME_CASES, EXTREMES

pytestmark = pytest.mark.gpu

ALGOS5 = ("returns", "gae", "td_lambda", "vtrace", "retrace")


def run_mat(algo, d, p, **kw):
    g = lambda k: d.get(k)
    if algo == "returns":
        res = {"returns": rl.rlca_returns_materialized(g("rewards"), g("terminated"),
                                                       g("truncated"), g("trunc_values"),
                                                       g("bootstrap"), gamma=p["gamma"], **kw)}
    elif algo == "gae":
        adv, tgt = rl.rlca_gae_materialized(g("rewards"), g("values"), g("terminated"),
                                            g("truncated"), g("trunc_values"), gamma=p["gamma"],
                                            lam=p["lam"], **kw)
        res = {"advantages": adv, "targets": tgt}
    elif algo == "td_lambda":
        res = {"lambda_returns": rl.rlca_td_lambda_materialized(
            g("rewards"), g("values"), g("terminated"), g("truncated"), g("trunc_values"),
            gamma=p["gamma"], lam=p["lam"], **kw)}
    elif algo == "vtrace":
        vs, pg = rl.rlca_vtrace_materialized(g("rewards"), g("values"), g("log_rhos"),
                                             g("terminated"), g("truncated"), g("trunc_values"),
                                             gamma=p["gamma"], lam=p["lam"],
                                             rho_bar=p["rho_bar"], c_bar=p["c_bar"],
                                             pg_rho_bar=p["pg_rho_bar"], **kw)
        res = {"vs": vs, "pg_advantages": pg}
    else:
        res = {"q_ret": rl.rlca_retrace_materialized(g("rewards"), g("q_taken"),
                                                     g("exp_q_next"), g("log_rhos"),
                                                     g("terminated"), g("truncated"),
                                                     gamma=p["gamma"], lam=p["lam"],
                                                     c_bar=p["c_bar"], **kw)}
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in res.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS5)
def test_materialized_matches_oracle(algo, dtype):
    p = params32(dict(DEFAULT_PARAMS, rho_bar=1.05, c_bar=0.95, pg_rho_bar=1.1))
    for N, T in ((1, 1), (3, 2), (5, 7), (9, 128), (4, 129), (6, 1000), (2, 4097)):
        for p_b in (0.05, 0.0):
            host = random_inputs(algo, N, T, 3000 + N + T, dtype, p_term=p_b, p_trunc=p_b)
            print(algo, dtype, "N", N, "T", T, "boundary rate", p_b, flush=True)
            got = run_mat(algo, to_device(host), p)
            assert_close(got, run_oracle(algo, host, p), TOL[dtype],
                         "%s/%s materialized %dx%d" % (algo, dtype, N, T))


@pytest.mark.parametrize("algo", ALGOS5)
def test_materialized_on_strided_rows_with_a_given_workspace(algo):
    p = params32(DEFAULT_PARAMS)
    N, T = 7, 300
    host = random_inputs(algo, N, T, 3100, "f32", p_term=0.02, p_trunc=0.02)
    dev = {}
    for k, v in to_device(host).items():
        if v.dim() == 2:
            buf = torch.full((N, v.shape[1] + 13), float("nan") if v.is_floating_point() else 1,
                             dtype=v.dtype, device="cuda")
            buf[:, :v.shape[1]] = v
            dev[k] = buf[:, :v.shape[1]]
        else:
            dev[k] = v
    ws = torch.full((rl.rlca_materialized_workspace_bytes(N, T) // 4,), float("nan"),
                    device="cuda")
    got = run_mat(algo, dev, p, workspace=ws)
    assert_close(got, run_oracle(algo, host, p), TOL["f32"], "%s/materialized strided" % algo)
    # and the fused call on the same inputs agrees to the same bar
    assert_close(got, run_gpu(algo, dev, p), TOL["f32"], "%s/materialized vs fused" % algo)


def _workload_case(name):
    w = WORKLOADS[name]
    host = make_workload(w)
    p = params32(dict(DEFAULT_PARAMS, gamma=w.gamma, lam=w.lam, **w.clips))
    return w, host, p


@pytest.mark.parametrize("name", ["returns_4x128", "gae_4096x128", "td_lambda_16384x256",
                                  "offpolicy_2048x1024", "gae_bf16_256x16384"])
def test_materialized_full_size_configs(name):
    w, host, p = _workload_case(name)
    algos = ("vtrace", "retrace") if w.algo == "vtrace+retrace" else (w.algo,)
    dev = to_device(host)
    for algo in algos:
        print(name, algo, flush=True)
        got = run_mat(algo, dev, p)
        assert_close(got, run_oracle(algo, host, p), TOL[w.dtype],
                     "%s/%s materialized full size" % (name, algo))


@pytest.mark.parametrize("algo,which", [c for c in EXTREME_CASES if c[0] in ALGOS5])
def test_materialized_parameter_extremes(algo, which):
    # The parameter extremes of the fused calls' test (gamma 0 and 1, lambda 0
    # and 1, infinite and tight ratio clips) through the doubling passes.
    p = params32(dict(DEFAULT_PARAMS, **EXTREMES[which]))
    host = random_inputs(algo, 12, 700, 3300 + which, "f32", p_term=0.01, p_trunc=0.005)
    got = run_mat(algo, to_device(host), p)
    assert_close(got, run_oracle(algo, host, p), TOL["f32"],
                 "%s materialized %s" % (algo, EXTREMES[which]))
