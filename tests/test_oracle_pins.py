"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle (``oracle/``) against one of:
  * a closed form of the recurrence (constant-gamma discounted sums),
  * a special case that reduces one algorithm to another,
  * the forward-view sum definitions in ``bruteforce.py`` (independent code),
  * exact rational arithmetic on the pages' affine operator,
  * the boundary invariants the rl-triton explainer states (Technical
    summary, Method 3): no signal crosses an episode boundary, termination
    and truncation differ, and the window bootstrap is counted once.
Inputs are seeded and synthetic.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import bruteforce as bf
import oracle

RTOL_BF = 1e-12   # oracle vs brute force: both fp64, different summation order


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if a.size else 0.0


def rand_inputs(seed, N, T, p_term=0.15, p_trunc=0.1, ratio_std=0.7):
    g = np.random.Generator(np.random.PCG64(seed))
    d = dict(
        r=g.standard_normal((N, T)),
        v=g.standard_normal((N, T + 1)),
        q=g.standard_normal((N, T)),
        eq=g.standard_normal((N, T)),
        lr=g.standard_normal((N, T)) * ratio_std,
        term=(g.random((N, T)) < p_term).astype(np.uint8),
        trunc=(g.random((N, T)) < p_trunc).astype(np.uint8),
        tv=g.standard_normal((N, T)),
        B=g.standard_normal(N),
    )
    return d


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.99, 1.0])
def test_returns_constant_reward_closed_form(gamma):
    T = 37
    r = np.ones((1, T))
    G = oracle.returns(r, gamma=gamma)[0]
    for t in range(T):
        n = T - t
        expect = n if gamma == 1.0 else (1 - gamma ** n) / (1 - gamma)
        assert abs(G[t] - expect) <= 1e-12 * max(1.0, expect)


def test_returns_one_hot_and_bootstrap_closed_form():
    T, gamma, j = 20, 0.9, 13
    r = np.zeros((1, T))
    r[0, j] = 1.0
    G = oracle.returns(r, bootstrap=np.array([0.0]), gamma=gamma)[0]
    for t in range(T):
        assert G[t] == pytest.approx(gamma ** (j - t) if t <= j else 0.0, abs=1e-15)
    # The bootstrap B enters once, discounted by gamma^{T-t}.
    G0 = oracle.returns(np.zeros((1, T)), bootstrap=np.array([2.0]), gamma=gamma)[0]
    for t in range(T):
        assert G0[t] == pytest.approx(2.0 * gamma ** (T - t), rel=1e-14)


def test_returns_no_dones_matches_discounted_sum():
    g = np.random.Generator(np.random.PCG64(7))
    N, T, gamma = 5, 64, 0.97
    r = g.standard_normal((N, T))
    B = g.standard_normal(N)
    G = oracle.returns(r, bootstrap=B, gamma=gamma)
    for n in range(N):
        for t in range(T):
            s = math.fsum(gamma ** k * r[n, t + k] for k in range(T - t)) + gamma ** (T - t) * B[n]
            assert abs(G[n, t] - s) <= 1e-12 * max(1.0, abs(s))


def test_termination_zeroes_successor_truncation_bootstraps():
    # A one-step episode after each flag: G_t = r_t (term), r_t + gamma*tv_t (trunc),
    # and termination wins when both are set.
    T, gamma = 4, 0.5
    r = np.array([[1.0, 2.0, 3.0, 4.0]])
    tv = np.array([[10.0, 20.0, 30.0, 40.0]])
    term = np.array([[1, 0, 1, 0]], np.uint8)
    trunc = np.array([[0, 1, 1, 0]], np.uint8)
    G = oracle.returns(r, term, trunc, tv, np.array([100.0]), gamma=gamma)[0]
    assert G[3] == 4.0 + 0.5 * 100.0
    assert G[2] == 3.0                       # term and trunc: termination wins
    assert G[1] == 2.0 + 0.5 * 20.0          # truncation: bootstrap tv_1
    assert G[0] == 1.0                       # termination: successor value 0


# ------------------------------------------------------- special-case reductions

def test_gae_special_cases():
    d = rand_inputs(11, 6, 40)
    kw = dict(terminated=d["term"], truncated=d["trunc"], trunc_values=d["tv"])
    gamma = 0.93
    # lam = 1: GAE advantage = discounted return (bootstrap V_T, same masks) - V_t.
    adv1, tgt1 = oracle.gae(d["r"], d["v"], gamma=gamma, lam=1.0, **kw)
    G = oracle.returns(d["r"], d["term"], d["trunc"], d["tv"], d["v"][:, -1], gamma=gamma)
    assert rel_err(adv1, G - d["v"][:, :-1]) < 1e-12
    assert rel_err(tgt1, G) < 1e-12
    # lam = 0: advantage = one-step TD error.
    adv0, _ = oracle.gae(d["r"], d["v"], gamma=gamma, lam=0.0, **kw)
    nv = np.where(d["term"] != 0, 0.0, np.where(d["trunc"] != 0, d["tv"], d["v"][:, 1:]))
    assert rel_err(adv0, d["r"] + gamma * nv - d["v"][:, :-1]) < 1e-15
    # gamma = 0: advantage = r - V.
    advg, _ = oracle.gae(d["r"], d["v"], gamma=0.0, lam=0.7, **kw)
    assert rel_err(advg, d["r"] - d["v"][:, :-1]) < 1e-15


def test_td_lambda_equals_gae_plus_values():
    # The oracle's TD(lambda) is a separate recursion (mixing V_{t+1} and G_{t+1});
    # it must agree with GAE + V.
    d = rand_inputs(12, 8, 50)
    kw = dict(terminated=d["term"], truncated=d["trunc"], trunc_values=d["tv"])
    for gamma, lam in [(0.99, 0.95), (0.5, 0.3), (1.0, 1.0), (0.9, 0.0)]:
        adv, tgt = oracle.gae(d["r"], d["v"], gamma=gamma, lam=lam, **kw)
        ret = oracle.td_lambda(d["r"], d["v"], gamma=gamma, lam=lam, **kw)
        assert rel_err(ret, adv + d["v"][:, :-1]) < 1e-13
        assert rel_err(ret, tgt) < 1e-13


def test_vtrace_reductions():
    d = rand_inputs(13, 6, 45)
    kw = dict(terminated=d["term"], truncated=d["trunc"], trunc_values=d["tv"])
    gamma, lam = 0.97, 0.8
    # On-policy (log ratio 0, clips 1): vs = TD(lambda) returns; pg = one-step TD target - V
    # with the next vs.
    vs, pg = oracle.vtrace(d["r"], d["v"], np.zeros_like(d["r"]), gamma=gamma, lam=lam, **kw)
    ret = oracle.td_lambda(d["r"], d["v"], gamma=gamma, lam=lam, **kw)
    assert rel_err(vs, ret) < 1e-13
    # lam = 0: vs_t = V_t + rho_t * delta_t.
    vs0, _ = oracle.vtrace(d["r"], d["v"], d["lr"], gamma=gamma, lam=0.0, **kw)
    rho = np.minimum(1.0, np.exp(d["lr"]))
    nv = np.where(d["term"] != 0, 0.0, np.where(d["trunc"] != 0, d["tv"], d["v"][:, 1:]))
    assert rel_err(vs0, d["v"][:, :-1] + rho * (d["r"] + gamma * nv - d["v"][:, :-1])) < 1e-14
    # Clipping: any log ratio >= 0 behaves exactly like log ratio 0 with clips 1.
    big = np.abs(d["lr"]) + 3.0
    vsb, pgb = oracle.vtrace(d["r"], d["v"], big, gamma=gamma, lam=lam, **kw)
    assert np.array_equal(vsb, vs) and np.array_equal(pgb, pg)


def test_retrace_reductions():
    d = rand_inputs(14, 6, 45)
    gamma, lam = 0.95, 0.9
    # lam = 0: Qret = r + gamma*(1-term)*EQ.
    q0 = oracle.retrace(d["r"], d["q"], d["eq"], d["lr"], d["term"], d["trunc"],
                        gamma=gamma, lam=0.0)
    assert rel_err(q0, d["r"] + gamma * (1 - d["term"]) * d["eq"]) < 1e-15
    # On-policy with EQ_t = Q_{t+1} (EQ_{T-1} = V_T, EQ_t = tv_t at truncations):
    # Retrace = TD(lambda) on the values [Q_0..Q_{T-1}, V_T].
    vals = np.concatenate([d["q"], d["v"][:, -1:]], axis=1)
    eq = vals[:, 1:].copy()
    eq = np.where(d["trunc"] != 0, d["tv"], eq)
    qr = oracle.retrace(d["r"], d["q"], eq, np.zeros_like(d["r"]), d["term"], d["trunc"],
                        gamma=gamma, lam=lam)
    ret = oracle.td_lambda(d["r"], vals, d["term"], d["trunc"], d["tv"], gamma=gamma, lam=lam)
    assert rel_err(qr, ret) < 1e-13


# ------------------------------------------------- forward-view brute force

@pytest.mark.parametrize("seed", [21, 22, 23])
@pytest.mark.parametrize("T", [1, 2, 5, 12])
def test_oracle_matches_forward_views(seed, T):
    N = 7
    d = rand_inputs(seed, N, T)
    gamma, lam = 0.9, 0.8
    tl = lambda a: a.tolist()
    term, trunc, tv = tl(d["term"]), tl(d["trunc"]), tl(d["tv"])

    G = oracle.returns(d["r"], d["term"], d["trunc"], d["tv"], d["B"], gamma=gamma)
    assert rel_err(G, bf.returns(tl(d["r"]), term, trunc, tv, tl(d["B"]), gamma)) < RTOL_BF

    adv, tgt = oracle.gae(d["r"], d["v"], d["term"], d["trunc"], d["tv"], gamma=gamma, lam=lam)
    adv_bf = np.array(bf.gae(tl(d["r"]), tl(d["v"]), term, trunc, tv, gamma, lam))
    assert rel_err(adv, adv_bf) < RTOL_BF
    assert rel_err(tgt, adv_bf + d["v"][:, :-1]) < RTOL_BF

    ret = oracle.td_lambda(d["r"], d["v"], d["term"], d["trunc"], d["tv"], gamma=gamma, lam=lam)
    assert rel_err(ret, bf.td_lambda(tl(d["r"]), tl(d["v"]), term, trunc, tv, gamma, lam)) < RTOL_BF

    clips = dict(rho_bar=1.1, c_bar=0.9, pg_rho_bar=1.3)
    vs, pg = oracle.vtrace(d["r"], d["v"], d["lr"], d["term"], d["trunc"], d["tv"],
                           gamma=gamma, lam=lam, **clips)
    vs_bf, pg_bf = bf.vtrace(tl(d["r"]), tl(d["v"]), tl(d["lr"]), term, trunc, tv, gamma, lam,
                             clips["rho_bar"], clips["c_bar"], clips["pg_rho_bar"])
    assert rel_err(vs, vs_bf) < RTOL_BF
    assert rel_err(pg, pg_bf) < RTOL_BF

    qr = oracle.retrace(d["r"], d["q"], d["eq"], d["lr"], d["term"], d["trunc"],
                        gamma=gamma, lam=lam, c_bar=0.9)
    qr_bf = bf.retrace(tl(d["r"]), tl(d["q"]), tl(d["eq"]), tl(d["lr"]), term, trunc,
                       gamma, lam, 0.9)
    assert rel_err(qr, qr_bf) < RTOL_BF


def test_trace_index_vtrace_from_t_retrace_from_t_plus_1():
    # With traces that vary per step, V-trace's product starts at c_t and
    # Retrace's at c_{t+1}; the brute force fixes which, the oracle must agree.
    T, gamma, lam = 3, 1.0, 1.0
    r = np.zeros((1, T))
    v = np.zeros((1, T + 1))
    v[0, T] = 1.0                      # only the window bootstrap is nonzero
    lr = np.log(np.array([[0.5, 0.25, 0.125]]))
    vs, _ = oracle.vtrace(r, v, lr, gamma=gamma, lam=lam, rho_bar=1.0, c_bar=1.0)
    # delta_2 = rho_2 * V_3 = 0.125; vs_0 = c_0 c_1 delta_2 = 0.5 * 0.25 * 0.125
    assert vs[0, 0] == pytest.approx(0.5 * 0.25 * 0.125, rel=1e-15)
    q = np.zeros((1, T))
    eq = np.array([[0.0, 0.0, 1.0]])
    qr = oracle.retrace(r, q, eq, lr, gamma=gamma, lam=lam, c_bar=1.0)
    # delta_2 = EQ_2 = 1; Qret_0 = c_1 c_2 * 1 = 0.25 * 0.125
    assert qr[0, 0] == pytest.approx(0.25 * 0.125, rel=1e-15)


# --------------------------------------- exhaustive boundary enumeration (T <= 6)

def all_boundary_patterns(T):
    """Every per-step state in {none, term, trunc, both}: 4^T rows."""
    pats = np.array(list(itertools.product(range(4), repeat=T)), dtype=np.int64)
    term = (pats & 1).astype(np.uint8)
    trunc = ((pats >> 1) & 1).astype(np.uint8)
    return term, trunc


@pytest.mark.parametrize("T", [1, 3, 5])
def test_exhaustive_boundaries_against_forward_views(T):
    term, trunc = all_boundary_patterns(T)
    N = term.shape[0]
    g = np.random.Generator(np.random.PCG64(1000 + T))
    r, v = g.standard_normal((N, T)), g.standard_normal((N, T + 1))
    tv, lr = g.standard_normal((N, T)), g.standard_normal((N, T)) * 0.5
    q, eq, B = g.standard_normal((N, T)), g.standard_normal((N, T)), g.standard_normal(N)
    gamma, lam = 0.9, 0.7
    tl = lambda a: a.tolist()
    t_, r_ = tl(term), tl(trunc)
    assert rel_err(oracle.returns(r, term, trunc, tv, B, gamma=gamma),
                   bf.returns(tl(r), t_, r_, tl(tv), tl(B), gamma)) < RTOL_BF
    adv, _ = oracle.gae(r, v, term, trunc, tv, gamma=gamma, lam=lam)
    assert rel_err(adv, bf.gae(tl(r), tl(v), t_, r_, tl(tv), gamma, lam)) < RTOL_BF
    assert rel_err(oracle.td_lambda(r, v, term, trunc, tv, gamma=gamma, lam=lam),
                   bf.td_lambda(tl(r), tl(v), t_, r_, tl(tv), gamma, lam)) < RTOL_BF
    vs, pg = oracle.vtrace(r, v, lr, term, trunc, tv, gamma=gamma, lam=lam,
                           rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0)
    vs_bf, pg_bf = bf.vtrace(tl(r), tl(v), tl(lr), t_, r_, tl(tv), gamma, lam, 1.0, 1.0, 1.0)
    assert rel_err(vs, vs_bf) < RTOL_BF and rel_err(pg, pg_bf) < RTOL_BF
    assert rel_err(oracle.retrace(r, q, eq, lr, term, trunc, gamma=gamma, lam=lam),
                   bf.retrace(tl(r), tl(q), tl(eq), tl(lr), t_, r_, gamma, lam, 1.0)) < RTOL_BF


# ------------------------------------------------------------------ invariants

def _all_outputs(d, gamma=0.95, lam=0.9):
    kw = dict(terminated=d["term"], truncated=d["trunc"], trunc_values=d["tv"])
    out = {"returns": oracle.returns(d["r"], d["term"], d["trunc"], d["tv"], d["B"], gamma=gamma)}
    out["adv"], out["tgt"] = oracle.gae(d["r"], d["v"], gamma=gamma, lam=lam, **kw)
    out["td"] = oracle.td_lambda(d["r"], d["v"], gamma=gamma, lam=lam, **kw)
    out["vs"], out["pg"] = oracle.vtrace(d["r"], d["v"], d["lr"], gamma=gamma, lam=lam, **kw)
    out["qret"] = oracle.retrace(d["r"], d["q"], d["eq"], d["lr"], d["term"], d["trunc"],
                                 gamma=gamma, lam=lam)
    return out


@pytest.mark.parametrize("kind", ["term", "trunc"])
def test_no_leak_across_episode_boundary(kind):
    # rl-triton, Method 3: signal stops at the boundary.  Perturb every input
    # after a boundary at step s (and the window bootstrap); outputs at t <= s
    # must be bitwise unchanged.
    N, T, s = 4, 30, 11
    d = rand_inputs(31, N, T, p_term=0.0, p_trunc=0.0)
    d[kind][:, s] = 1
    base = _all_outputs(d)
    p = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    g = np.random.Generator(np.random.PCG64(32))
    for k in ("r", "q", "eq", "lr", "tv"):
        p[k][:, s + 1:] = g.standard_normal((N, T - s - 1)) * 5
    p["v"][:, s + 2:] = g.standard_normal((N, T - s - 1)) * 5   # V_{s+2}..V_T
    p["B"] = p["B"] + 7.0
    if kind == "term":
        # After a termination even V_{s+1} and tv_s are unused.
        p["v"][:, s + 1] += 3.0
        p["tv"][:, s] += 3.0
    else:
        # After a truncation V_{s+1} belongs to the next episode and is unused.
        p["v"][:, s + 1] += 3.0
    pert = _all_outputs(p)
    for name in base:
        assert np.array_equal(base[name][:, : s + 1], pert[name][:, : s + 1]), name


def test_window_bootstrap_counted_once_and_ignored_after_done():
    # rl-triton, Method 3 (rollout windows): with no boundary, the bootstrap V_T
    # enters A_{T-1} once: A_{T-1} = r + gamma*V_T - V_{T-1}.
    N, T, gamma, lam = 3, 9, 0.9, 0.8
    d = rand_inputs(41, N, T, p_term=0.0, p_trunc=0.0)
    adv, _ = oracle.gae(d["r"], d["v"], gamma=gamma, lam=lam)
    assert np.allclose(adv[:, -1], d["r"][:, -1] + gamma * d["v"][:, -1] - d["v"][:, -2],
                       rtol=0, atol=1e-15)
    G = oracle.returns(d["r"], bootstrap=d["B"], gamma=gamma)
    assert np.allclose(G[:, -1], d["r"][:, -1] + gamma * d["B"], rtol=0, atol=1e-15)
    # If the last step is a boundary, the window bootstrap has no effect.
    for kind in ("term", "trunc"):
        e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
        e[kind][:, -1] = 1
        a = _all_outputs(e)
        e["v"][:, -1] += 11.0
        e["B"] = e["B"] - 5.0
        b = _all_outputs(e)
        for name in a:
            assert np.array_equal(a[name], b[name]), (kind, name)


def test_linearity_in_rewards_and_values():
    # Scaling every additive input by 2 scales every output by exactly 2
    # (powers of two are exact in binary floating point).
    d = rand_inputs(51, 4, 33)
    e = {k: v for k, v in d.items()}
    for k in ("r", "v", "q", "eq", "tv", "B"):
        e[k] = d[k] * 2.0
    a, b = _all_outputs(d), _all_outputs(e)
    for name in a:
        assert np.array_equal(2.0 * a[name], b[name]), name


def test_rows_are_independent():
    d = rand_inputs(61, 9, 17)
    perm = np.random.Generator(np.random.PCG64(62)).permutation(9)
    e = {k: v[perm] for k, v in d.items()}
    a, b = _all_outputs(d), _all_outputs(e)
    for name in a:
        assert np.array_equal(a[name][perm], b[name]), name


# ------------------------------------------- the pages' affine operator, exactly

def _oplus(B, A):
    """(alpha_B, beta_B) (+) (alpha_A, beta_A) = (alpha_B + beta_B alpha_A, beta_A beta_B);
    rl-triton, Method 1.  B is the earlier step."""
    return (B[0] + B[1] * A[0], A[1] * B[1])


def _tree_scan(pairs, rng):
    """Composite of pairs[0] (+) ... (+) pairs[-1] by a random bracketing."""
    if len(pairs) == 1:
        return pairs[0]
    k = rng.integers(1, len(pairs))
    return _oplus(_tree_scan(pairs[:k], rng), _tree_scan(pairs[k:], rng))


def test_affine_operator_scan_equals_gae_recurrence_exactly():
    # Any bracketing of the operator gives exactly (rational arithmetic) the
    # oracle's backward GAE recursion, with alpha_t = delta_t and
    # beta_t = gamma*lam*(1 - done_t), carry A_T = 0.
    rng = np.random.Generator(np.random.PCG64(71))
    T = 9
    gamma, lam = Fraction(9, 10), Fraction(3, 4)
    for trial in range(20):
        r = [Fraction(int(x), 8) for x in rng.integers(-16, 17, T)]
        v = [Fraction(int(x), 4) for x in rng.integers(-8, 9, T + 1)]
        tv = [Fraction(int(x), 4) for x in rng.integers(-8, 9, T)]
        term = [int(x) for x in (rng.random(T) < 0.2)]
        trunc = [int(x) for x in (rng.random(T) < 0.2)]
        alpha, beta = [], []
        for t in range(T):
            succ = 0 if term[t] else (tv[t] if trunc[t] else v[t + 1])
            alpha.append(r[t] + gamma * succ - v[t])
            beta.append(gamma * lam * (0 if (term[t] or trunc[t]) else 1))
        ref, _ = oracle.gae(np.array([[float(x) for x in r]]), np.array([[float(x) for x in v]]),
                            np.array([term], np.uint8), np.array([trunc], np.uint8),
                            np.array([[float(x) for x in tv]]), gamma=float(gamma), lam=float(lam))
        for t in range(T):
            a, b = _tree_scan(list(zip(alpha[t:], beta[t:])), rng)
            A_t = a + b * 0           # carry A_T = 0
            assert abs(float(A_t) - ref[0, t]) <= 1e-13 * max(1.0, abs(float(A_t)))


# ------------------------------------------------------- regression fixture

def test_oracle_regression_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "oracle_regression.json")
    with open(path) as f:
        doc = json.load(f)
    i = {k: np.array(v) for k, v in doc["inputs"].items()}
    p = doc["params"]
    term, trunc = i["term"].astype(np.uint8), i["trunc"].astype(np.uint8)
    got = {"returns": oracle.returns(i["r"], term, trunc, i["tv"], i["B"], gamma=p["gamma"])}
    got["adv"], got["tgt"] = oracle.gae(i["r"], i["v"], term, trunc, i["tv"],
                                        gamma=p["gamma"], lam=p["lam"])
    got["td_lambda"] = oracle.td_lambda(i["r"], i["v"], term, trunc, i["tv"],
                                        gamma=p["gamma"], lam=p["lam"])
    got["vs"], got["pg"] = oracle.vtrace(i["r"], i["v"], i["lr"], term, trunc, i["tv"],
                                         gamma=p["gamma"], lam=p["lam"], rho_bar=p["rho_bar"],
                                         c_bar=p["c_bar"], pg_rho_bar=p["pg_rho_bar"])
    got["qret"] = oracle.retrace(i["r"], i["q"], i["eq"], i["lr"], term, trunc,
                                 gamma=p["gamma"], lam=p["lam"], c_bar=p["c_bar"])
    got["eligibility"] = oracle.eligibility_trace(i["r"], term, trunc, i["B"], gamma=p["gamma"],
                                                  lam=p["lam"])
    got["cumsum"] = oracle.episodic_cumsum(i["r"], term, trunc, i["B"])
    for k, rows in doc["outputs"].items():
        want = np.array([[float.fromhex(x) for x in row] for row in rows])
        assert rel_err(got[k], want) < 1e-15, k


# -------------------------------------------- forward-time mirrors (eq. R forward)

def test_forward_recurrences_without_boundaries_are_library_cumsums():
    g = np.random.Generator(np.random.PCG64(81))
    x = g.standard_normal((5, 40))
    # Plain prefix sum: numpy's cumsum.
    assert rel_err(oracle.episodic_cumsum(x), np.cumsum(x, axis=1)) < 1e-13
    # Carry-in adds to every step of the first episode.
    s0 = g.standard_normal(5)
    assert rel_err(oracle.episodic_cumsum(x, s_init=s0), np.cumsum(x, axis=1) + s0[:, None]) < 1e-13
    # Constant input, geometric decay: z_t = (1 - d^{t+1}) / (1 - d).
    d = 0.9 * 0.8
    z = oracle.eligibility_trace(np.ones((1, 30)), gamma=0.9, lam=0.8)[0]
    for t in range(30):
        assert z[t] == pytest.approx((1 - d ** (t + 1)) / (1 - d), rel=1e-14)
    # gamma*lam = 1 reduces the trace to the prefix sum.
    assert rel_err(oracle.eligibility_trace(x, gamma=1.0, lam=1.0), np.cumsum(x, axis=1)) < 1e-13


def test_forward_boundary_restarts_next_step():
    # A boundary after step 2 restarts at step 3; termination and truncation
    # act the same for forward recurrences.
    x = np.array([[1.0, 2.0, 3.0, 4.0, 5.0]])
    for kind in ("term", "trunc"):
        f = np.zeros((1, 5), np.uint8)
        f[0, 2] = 1
        kw = {"terminated": f} if kind == "term" else {"truncated": f}
        s = oracle.episodic_cumsum(x, s_init=np.array([10.0]), **kw)[0]
        assert list(s) == [11.0, 13.0, 16.0, 4.0, 9.0]


@pytest.mark.parametrize("seed", [82, 83])
@pytest.mark.parametrize("T", [1, 4, 13])
def test_forward_oracle_matches_forward_sums(seed, T):
    d = rand_inputs(seed, 6, T)
    tl = lambda a: a.tolist()
    z = oracle.eligibility_trace(d["r"], d["term"], d["trunc"], d["B"], gamma=0.9, lam=0.7)
    zb = bf.eligibility_trace(tl(d["r"]), tl(d["term"]), tl(d["trunc"]), tl(d["B"]), 0.9 * 0.7)
    assert rel_err(z, zb) < RTOL_BF
    s = oracle.episodic_cumsum(d["r"], d["term"], d["trunc"], d["B"])
    sb = bf.episodic_cumsum(tl(d["r"]), tl(d["term"]), tl(d["trunc"]), tl(d["B"]))
    assert rel_err(s, sb) < RTOL_BF


def test_forward_exhaustive_boundaries():
    term, trunc = all_boundary_patterns(5)
    N = term.shape[0]
    g = np.random.Generator(np.random.PCG64(84))
    x, z0 = g.standard_normal((N, 5)), g.standard_normal(N)
    tl = lambda a: a.tolist()
    assert rel_err(oracle.eligibility_trace(x, term, trunc, z0, gamma=0.95, lam=0.5),
                   bf.eligibility_trace(tl(x), tl(term), tl(trunc), tl(z0), 0.95 * 0.5)) < RTOL_BF
    assert rel_err(oracle.episodic_cumsum(x, term, trunc, z0),
                   bf.episodic_cumsum(tl(x), tl(term), tl(trunc), tl(z0))) < RTOL_BF


def test_forward_no_leak_bitwise():
    # A boundary after step s: perturbing inputs at steps <= s (and the
    # carry-in) leaves outputs at steps > s bitwise unchanged.
    d = rand_inputs(85, 4, 30, p_term=0.0, p_trunc=0.0)
    s = 12
    for kind in ("term", "trunc"):
        f = np.zeros((4, 30), np.uint8)
        f[:, s] = 1
        kw = {"terminated": f} if kind == "term" else {"truncated": f}
        x2 = d["r"].copy()
        x2[:, : s + 1] += 5.0
        for fn, extra in ((oracle.episodic_cumsum, {}),
                          (oracle.eligibility_trace, {"gamma": 0.9, "lam": 0.9})):
            a = fn(d["r"], s_init=d["B"], **kw, **extra) if fn is oracle.episodic_cumsum else \
                fn(d["r"], z_init=d["B"], **kw, **extra)
            b = fn(x2, s_init=d["B"] + 3, **kw, **extra) if fn is oracle.episodic_cumsum else \
                fn(x2, z_init=d["B"] + 3, **kw, **extra)
            assert np.array_equal(a[:, s + 1:], b[:, s + 1:]), (kind, fn.__name__)


# ------------------------------------- window carries (Method 3, rollout windows)

CARRY_KINDS = ("returns", "gae", "td_lambda", "vtrace", "retrace", "eligibility", "cumsum")
FORWARD_KINDS = ("eligibility", "cumsum")
WP = dict(gamma=0.93, lam=0.85, rho_bar=1.1, c_bar=0.9, pg_rho_bar=1.3)


def run_window(kind, d, lo, hi, carry, p=WP):
    """One window [lo, hi) of the rollout in ``d``: (outputs, carry_out, carry_map)."""
    s = slice(lo, hi)
    r, te, tr, tv = d["r"][:, s], d["term"][:, s], d["trunc"][:, s], d["tv"][:, s]
    v = d["v"][:, lo:hi + 1]
    g, lam = p["gamma"], p["lam"]
    if kind == "returns":
        G, co, cm = oracle.returns(r, te, tr, tv, carry, gamma=g, chunk=True)
        return (G,), co, cm
    if kind == "gae":
        a, tg, co, cm = oracle.gae(r, v, te, tr, tv, gamma=g, lam=lam, carry_in=carry, chunk=True)
        return (a, tg), co, cm
    if kind == "td_lambda":
        G, co, cm = oracle.td_lambda(r, v, te, tr, tv, gamma=g, lam=lam, carry_in=carry,
                                     chunk=True)
        return (G,), co, cm
    if kind == "vtrace":
        vs, pg, co, cm = oracle.vtrace(r, v, d["lr"][:, s], te, tr, tv, gamma=g, lam=lam,
                                       rho_bar=p["rho_bar"], c_bar=p["c_bar"],
                                       pg_rho_bar=p["pg_rho_bar"], carry_in=carry, chunk=True)
        return (vs, pg), co, cm
    if kind == "retrace":
        q, co, cm = oracle.retrace(r, d["q"][:, s], d["eq"][:, s], d["lr"][:, s], te, tr,
                                   gamma=g, lam=lam, c_bar=p["c_bar"], carry_in=carry, chunk=True)
        return (q,), co, cm
    if kind == "eligibility":
        z, co, cm = oracle.eligibility_trace(r, te, tr, carry, gamma=g, lam=lam, chunk=True)
        return (z,), co, cm
    S, co, cm = oracle.episodic_cumsum(r, te, tr, carry, chunk=True)
    return (S,), co, cm


def _boundaries_at(d, k):
    """Force each kind of boundary right before and at the cut k."""
    d = {key: (val.copy() if hasattr(val, "copy") else val) for key, val in d.items()}
    d["term"][0, k - 1], d["trunc"][0, k - 1] = 1, 0
    d["term"][1, k - 1], d["trunc"][1, k - 1] = 0, 1
    d["term"][2, k], d["trunc"][2, k] = 1, 0
    d["term"][3, k], d["trunc"][3, k] = 0, 1
    d["term"][4, k - 1: k + 1] = 0
    d["trunc"][4, k - 1: k + 1] = 0
    return d


@pytest.mark.parametrize("kind", CARRY_KINDS)
@pytest.mark.parametrize("seed", [91, 92])
def test_window_split_reproduces_one_long_window(kind, seed):
    # Cutting a rollout at k and chaining the two windows through
    # carry_out -> carry_in gives the result of the uncut window (whose
    # definition the pins above fix).
    N, T = 8, 23
    for k in (1, 7, 22):
        d = _boundaries_at(rand_inputs(seed, N, T), k)
        first = d["B"] if kind in FORWARD_KINDS else None
        whole, whole_co, _ = run_window(kind, d, 0, T, first)
        if kind in FORWARD_KINDS:
            e_out, e_co, _ = run_window(kind, d, 0, k, first)
            l_out, l_co, _ = run_window(kind, d, k, T, e_co)
            chained_co = l_co
        else:
            l_out, l_co, _ = run_window(kind, d, k, T, None)
            e_out, e_co, _ = run_window(kind, d, 0, k, l_co)
            chained_co = e_co
        for w, e, l in zip(whole, e_out, l_out):
            assert rel_err(np.concatenate([e, l], axis=1), w) < 1e-12, (kind, k)
        assert rel_err(chained_co, whole_co) < 1e-12, (kind, k)


@pytest.mark.parametrize("kind", CARRY_KINDS)
def test_carry_map_is_the_affine_map_of_the_carry(kind):
    # Few boundaries, so that most rows carry through the whole window.
    d = rand_inputs(93, 6, 17, p_term=0.03, p_trunc=0.02)
    _, co0, m0 = run_window(kind, d, 0, 17, None)
    assert np.array_equal(m0[:, 0], co0)  # a = carry_out from carry 0
    for x in (0.75, -1.5, 40.0):
        c = np.full(6, x) + d["B"]
        _, co, m = run_window(kind, d, 0, 17, c)
        assert np.array_equal(m, m0)  # the map does not depend on the carry
        assert rel_err(co, m[:, 0] + m[:, 1] * c) < 1e-12


@pytest.mark.parametrize("kind", CARRY_KINDS)
def test_carry_map_closed_forms(kind):
    # No boundaries, log-ratios 0 (every clipped ratio is 1, c_t = lam):
    # b is the product of the per-step factors, (gamma*lam)^T, gamma^T for
    # returns and 1 for the plain prefix sum.
    N, T = 3, 9
    d = rand_inputs(94, N, T, p_term=0.0, p_trunc=0.0)
    d["lr"][:] = 0.0
    g, lam = WP["gamma"], WP["lam"]
    want_b = {"returns": g ** T, "cumsum": 1.0}.get(kind, (g * lam) ** T)
    _, _, m = run_window(kind, d, 0, T, None, p=dict(WP, c_bar=1.0, rho_bar=1.0))
    assert np.allclose(m[:, 1], want_b, rtol=1e-13, atol=0)
    # A boundary anywhere before the window's last step cuts the carry: b = 0
    # (reverse: any step; forward: any step but the last) ...
    for j in (0, 4, T - 1):
        for flag in ("term", "trunc"):
            e = {key: (val.copy() if hasattr(val, "copy") else val) for key, val in d.items()}
            e[flag][:, j] = 1
            _, co, m = run_window(kind, e, 0, T, None)
            assert np.all(m[:, 1] == 0.0), (kind, j, flag)
            if kind in FORWARD_KINDS and j == T - 1:
                # ... and a boundary after the last step passes nothing on.
                assert np.all(co == 0.0) and np.all(m == 0.0)


def test_carry_closed_forms_one_step():
    # T = 1, no boundary: the carry enters exactly where the published
    # recursions put the quantity of the step after the window.
    g, lam = WP["gamma"], WP["lam"]
    d = rand_inputs(95, 5, 1, p_term=0.0, p_trunc=0.0)
    c = np.array([0.3, -1.2, 2.0, 0.0, 5.5])
    r, v0, v1 = d["r"][:, 0], d["v"][:, 0], d["v"][:, 1]
    (a, tg), co, _ = run_window("gae", d, 0, 1, c)
    assert rel_err(a[:, 0], r + g * v1 - v0 + g * lam * c) < 1e-14
    assert rel_err(co, a[:, 0]) == 0
    (G,), co, _ = run_window("td_lambda", d, 0, 1, c)
    assert rel_err(G[:, 0], r + g * ((1 - lam) * v1 + lam * (v1 + c))) < 1e-14
    assert rel_err(co, G[:, 0] - v0) < 1e-14
    ratio = np.exp(d["lr"][:, 0])
    rho, cc = np.minimum(WP["rho_bar"], ratio), lam * np.minimum(WP["c_bar"], ratio)
    (vs, pg), co, _ = run_window("vtrace", d, 0, 1, c)
    assert rel_err(vs[:, 0], v0 + rho * (r + g * v1 - v0) + g * cc * c) < 1e-14
    assert rel_err(pg[:, 0], np.minimum(WP["pg_rho_bar"], ratio) * (r + g * (v1 + c) - v0)) < 1e-14
    assert rel_err(co, vs[:, 0] - v0) < 1e-14
    (Q,), co, _ = run_window("retrace", d, 0, 1, c)
    assert rel_err(Q[:, 0], r + g * d["eq"][:, 0] + g * c) < 1e-14
    assert rel_err(co, cc * (Q[:, 0] - d["q"][:, 0])) < 1e-14
    (z,), co, _ = run_window("eligibility", d, 0, 1, c)
    assert rel_err(z[:, 0], r + g * lam * c) < 1e-14 and rel_err(co, z[:, 0]) == 0


@pytest.mark.parametrize("kind", CARRY_KINDS)
def test_windows_evaluated_apart_chain_through_their_maps(kind):
    # The T-split: every window runs from carry 0 and reports its map; the
    # maps, composed from the far end, give each window's true carry; a second
    # pass with those carries reproduces the uncut window.
    N, T = 7, 40
    d = rand_inputs(96, N, T, p_term=0.04, p_trunc=0.03)
    cuts = [0, 9, 10, 26, 40]
    first = d["B"] if kind in FORWARD_KINDS else None
    whole, whole_co, _ = run_window(kind, d, 0, T, first)
    wins = list(zip(cuts[:-1], cuts[1:]))
    maps = [run_window(kind, d, lo, hi, None)[2] for lo, hi in wins]
    carries = [None] * len(wins)
    order = range(len(wins)) if kind in FORWARD_KINDS else range(len(wins) - 1, -1, -1)
    c = first if first is not None else np.zeros(N)
    for i in order:
        carries[i] = c
        c = maps[i][:, 0] + maps[i][:, 1] * c
    assert rel_err(c, whole_co) < 1e-12
    outs = [run_window(kind, d, lo, hi, carries[i])[0] for i, (lo, hi) in enumerate(wins)]
    for j, w in enumerate(whole):
        assert rel_err(np.concatenate([o[j] for o in outs], axis=1), w) < 1e-12, kind


# ------------------------------------------ generic segmented affine scan (eq. R)

@pytest.mark.parametrize("reverse", [True, False])
def test_affine_scan_constant_beta_is_a_first_order_iir_filter(reverse):
    # y_t = x_t + b y_{t-1} is scipy's lfilter([1], [1, -b]); the carry is the
    # filter state y_{-1}, i.e. initial condition zi = b * carry.
    from scipy.signal import lfilter
    g = np.random.Generator(np.random.PCG64(97))
    N, T, b = 4, 50, 0.97
    x, c = g.standard_normal((N, T)), g.standard_normal(N)
    A, co, m = oracle.affine_scan(x, np.full((N, T), b), carry_in=c, reverse=reverse)
    for n in range(N):
        xs = x[n, ::-1] if reverse else x[n]
        y, _ = lfilter([1.0], [1.0, -b], xs, zi=[b * c[n]])
        want = y[::-1] if reverse else y
        assert rel_err(A[n], want) < 1e-13
    assert rel_err(co, A[:, 0] if reverse else A[:, -1]) == 0
    assert np.allclose(m[:, 1], b ** T, rtol=1e-13, atol=0)


def test_affine_scan_unit_beta_is_cumsum():
    g = np.random.Generator(np.random.PCG64(98))
    x, c = g.standard_normal((3, 31)), g.standard_normal(3)
    A, _, _ = oracle.affine_scan(x, np.ones((3, 31)), carry_in=c, reverse=False)
    assert rel_err(A, np.cumsum(x, axis=1) + c[:, None]) < 1e-13
    A, _, _ = oracle.affine_scan(x, np.ones((3, 31)), carry_in=c, reverse=True)
    assert rel_err(A, np.cumsum(x[:, ::-1], axis=1)[:, ::-1] + c[:, None]) < 1e-13


@pytest.mark.parametrize("reverse", [True, False])
@pytest.mark.parametrize("seed,T", [(99, 1), (100, 6), (101, 15)])
def test_affine_scan_matches_sum_form(reverse, seed, T):
    g = np.random.Generator(np.random.PCG64(seed))
    N = 5
    al, be = g.standard_normal((N, T)), g.uniform(-1.2, 1.2, (N, T))
    rs = (g.random((N, T)) < 0.2).astype(np.uint8)
    c = g.standard_normal(N)
    A, co, m = oracle.affine_scan(al, be, rs, c, reverse=reverse)
    want = bf.affine_scan(al.tolist(), be.tolist(), rs.tolist(), c.tolist(), reverse)
    assert rel_err(A, want) < RTOL_BF
    want0 = bf.affine_scan(al.tolist(), be.tolist(), rs.tolist(), None, reverse)
    assert rel_err(m[:, 0], [row[0] if reverse else row[-1] for row in want0]) < RTOL_BF


@pytest.mark.parametrize("reverse", [True, False])
def test_affine_scan_exhaustive_resets(reverse):
    T = 5
    pats = np.array(list(itertools.product([0, 1], repeat=T)), np.uint8)
    N = len(pats)
    g = np.random.Generator(np.random.PCG64(102))
    al, be, c = g.standard_normal((N, T)), g.uniform(0.5, 1.5, (N, T)), g.standard_normal(N)
    A, _, _ = oracle.affine_scan(al, be, pats, c, reverse=reverse)
    assert rel_err(A, bf.affine_scan(al.tolist(), be.tolist(), pats.tolist(), c.tolist(),
                                     reverse)) < RTOL_BF


def test_affine_scan_exact_in_rationals():
    # Small integer/dyadic inputs: the fp64 result is exact and equals the
    # sum form evaluated in Fractions.
    al = [[3, -1, 4, 1, -5, 9]]
    be = [[0.5, 0.25, 2.0, -1.0, 0.5, 1.0]]
    rs = [[0, 0, 1, 0, 0, 0]]
    for reverse in (True, False):
        A, _, _ = oracle.affine_scan(np.array(al, float), np.array(be), np.array(rs, np.uint8),
                                     np.array([2.0]), reverse=reverse)
        want = bf.affine_scan([[Fraction(x) for x in al[0]]],
                              [[Fraction(x) for x in be[0]]], rs, [Fraction(2)], reverse)
        assert [Fraction(x) for x in A[0]] == want[0]


def test_affine_scan_instances_of_the_algorithms():
    # GAE is the reverse scan with alpha = delta and beta = gamma*lam cut at
    # done; the eligibility trace is the forward scan cut after done_{t-1}.
    d = rand_inputs(103, 6, 20)
    g, lam = 0.95, 0.9
    te, tr = d["term"].astype(bool), d["trunc"].astype(bool)
    nv = np.where(te, 0.0, np.where(tr, d["tv"], d["v"][:, 1:]))
    delta = d["r"] + g * nv - d["v"][:, :-1]
    A, _, _ = oracle.affine_scan(delta, np.full((6, 20), g * lam), (te | tr).astype(np.uint8))
    assert rel_err(A, oracle.gae(d["r"], d["v"], d["term"], d["trunc"], d["tv"], gamma=g,
                                 lam=lam)[0]) < 1e-13
    prev_done = np.zeros_like(te)
    prev_done[:, 1:] = (te | tr)[:, :-1]
    Z, _, _ = oracle.affine_scan(d["r"], np.full((6, 20), g * lam), prev_done.astype(np.uint8),
                                 d["B"], reverse=False)
    assert rel_err(Z, oracle.eligibility_trace(d["r"], d["term"], d["trunc"], d["B"], gamma=g,
                                               lam=lam)) < 1e-13


# --------------------- Retrace and V-trace from policy tables (Results section)

def _log_softmax(x):
    m = x.max(-1, keepdims=True)
    return x - m - np.log(np.exp(x - m).sum(-1, keepdims=True))


def prob_tables(seed, N, T, A, p_term=0.1, p_trunc=0.1):
    d = rand_inputs(seed, N, T, p_term=p_term, p_trunc=p_trunc)
    g = np.random.Generator(np.random.PCG64(seed + 1000))
    d["Q"] = g.standard_normal((N, T + 1, A))
    d["logpi"] = _log_softmax(g.standard_normal((N, T + 1, A)))
    d["logmu"] = _log_softmax(g.standard_normal((N, T, A)))
    d["act"] = g.integers(0, A, (N, T)).astype(np.int32)
    d["teq"] = g.standard_normal((N, T))
    return d


def _taken(table, act):
    return np.take_along_axis(table, act[..., None].astype(np.int64), -1)[..., 0]


PP = dict(gamma=0.95, lam=0.9, c_bar=0.9)


def _retrace_probs(d, **kw):
    return oracle.retrace_probs(d["r"], d["Q"], d["act"], d["logpi"], d["logmu"], d["term"],
                                d["trunc"], d["teq"], **dict(PP, **kw))


@pytest.mark.parametrize("seed,A", [(111, 1), (112, 4), (113, 18)])
def test_retrace_probs_is_retrace_of_the_table_quantities(seed, A):
    # q_taken, E_pi Q(s_{t+1}) and the log-ratio formed here with numpy from
    # their definitions, then the (pinned) Retrace oracle.
    N, T = 5, 21
    d = prob_tables(seed, N, T, A)
    T_ = d["r"].shape[1]
    q_taken = _taken(d["Q"][:, :T_], d["act"])
    eq = (np.exp(d["logpi"][:, 1:]) * d["Q"][:, 1:]).sum(-1)
    trunc_only = d["trunc"].astype(bool) & ~d["term"].astype(bool)
    eq = np.where(trunc_only, d["teq"], eq)
    lr = _taken(d["logpi"][:, :T_], d["act"]) - _taken(d["logmu"], d["act"])
    want = oracle.retrace(d["r"], q_taken, eq, lr, d["term"], d["trunc"], **PP)
    assert rel_err(_retrace_probs(d), want) < 1e-13


@pytest.mark.parametrize("seed,A", [(114, 1), (115, 6)])
def test_vtrace_probs_is_vtrace_of_the_table_ratio(seed, A):
    N, T = 4, 17
    d = prob_tables(seed, N, T, A)
    lr = _taken(d["logpi"][:, :T], d["act"]) - _taken(d["logmu"], d["act"])
    kw = dict(gamma=0.97, lam=0.9, rho_bar=1.2, c_bar=0.8, pg_rho_bar=1.1)
    want = oracle.vtrace(d["r"], d["v"], lr, d["term"], d["trunc"], d["tv"], **kw)
    got = oracle.vtrace_probs(d["r"], d["v"], d["act"], d["logpi"][:, :T], d["logmu"],
                              d["term"], d["trunc"], d["tv"], **kw)
    for a, b in zip(got, want):
        assert rel_err(a, b) < 1e-13


def test_retrace_probs_single_action_and_greedy_target():
    # One action: pi = 1, so E_pi Q(s_{t+1}) = Q(s_{t+1}, 0) and the ratio is
    # 1 / mu.  A greedy target policy makes E_pi Q the maximum over actions.
    N, T = 3, 12
    d = prob_tables(116, N, T, 1, p_term=0.0, p_trunc=0.0)
    d["logpi"][:] = 0.0
    d["logmu"][:] = np.log(0.5)
    lam_c = min(0.9, 2.0) * 0.9
    want = oracle.retrace(d["r"], d["Q"][:, :T, 0], d["Q"][:, 1:, 0],
                          np.full((N, T), np.log(2.0)), **PP)
    assert rel_err(_retrace_probs(d), want) < 1e-13
    d = prob_tables(117, N, T, 7, p_term=0.0, p_trunc=0.0)
    best = d["Q"].argmax(-1)
    with np.errstate(divide="ignore"):
        d["logpi"] = np.where(np.arange(7) == best[..., None], 0.0, -np.inf)
    q_taken = _taken(d["Q"][:, :T], d["act"])
    lr = _taken(d["logpi"][:, :T], d["act"]) - _taken(d["logmu"], d["act"])
    want = oracle.retrace(d["r"], q_taken, d["Q"][:, 1:].max(-1), lr, **PP)
    got = _retrace_probs(d)
    assert np.all(np.isfinite(got)) and rel_err(got, want) < 1e-13
    assert lam_c > 0


def test_probs_action_relabeling_is_invariant():
    N, T, A = 4, 15, 9
    d = prob_tables(118, N, T, A)
    perm = np.random.Generator(np.random.PCG64(119)).permutation(A)
    inv = np.argsort(perm)
    e = dict(d, Q=d["Q"][..., perm], logpi=d["logpi"][..., perm], logmu=d["logmu"][..., perm],
             act=inv[d["act"]].astype(np.int32))
    assert rel_err(_retrace_probs(e), _retrace_probs(d)) < 1e-14
    kw = dict(gamma=0.9, lam=0.95)
    a = oracle.vtrace_probs(d["r"], d["v"], d["act"], d["logpi"][:, :T], d["logmu"], **kw)
    b = oracle.vtrace_probs(e["r"], e["v"], e["act"], e["logpi"][:, :T], e["logmu"], **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_probs_tables_are_read_only_where_the_definition_reads_them():
    N, T, A = 3, 10, 5
    d = prob_tables(120, N, T, A, p_term=0.0, p_trunc=0.0)
    base = _retrace_probs(d)
    # Slice 0 enters only through the taken action (q_taken_0, log_rho_0).
    e = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in d.items()}
    others = np.arange(A)[None, :] != d["act"][:, :1]
    e["Q"][:, 0][others] += 7.0
    e["logpi"][:, 0][others] -= 3.0
    e["logmu"][others[:, None, :].repeat(T, 1) & (np.arange(T)[None, :, None] == 0)] += 1.0
    assert np.array_equal(_retrace_probs(e), base)
    # After a truncation at step s the expectation comes from trunc_eq, and
    # the trace is cut: slice s+1 then reaches no output at or before s.
    # (Without the truncation the same change moves step s.)
    s = 4
    noise = np.random.Generator(np.random.PCG64(122)).standard_normal((N, A))
    e = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in d.items()}
    e["Q"][:, s + 1] += 5.0
    e["logpi"][:, s + 1] = _log_softmax(e["logpi"][:, s + 1] + noise)
    assert not np.array_equal(_retrace_probs(e)[:, s], _retrace_probs(d)[:, s])
    d["trunc"][:, s] = 1
    e["trunc"] = d["trunc"]
    assert np.array_equal(_retrace_probs(e)[:, : s + 1], _retrace_probs(d)[:, : s + 1])


def test_probs_reject_actions_out_of_range():
    d = prob_tables(121, 2, 5, 3)
    for bad in (-1, 3):
        e = dict(d, act=d["act"].copy())
        e["act"][1, 2] = bad
        with pytest.raises(ValueError):
            _retrace_probs(e)


def test_probs_taken_behaviour_entries_equal_the_table_form():
    # log_mu given as the taken actions' entries [N, T] equals the table form
    # bitwise (the same numbers enter); the table's other entries are unread.
    N, T, A = 4, 13, 6
    d = prob_tables(123, N, T, A)
    taken = _taken(d["logmu"], d["act"])
    e = dict(d, logmu=taken)
    assert np.array_equal(_retrace_probs(e), _retrace_probs(d))
    kw = dict(gamma=0.9, lam=0.95)
    a = oracle.vtrace_probs(d["r"], d["v"], d["act"], d["logpi"][:, :T], d["logmu"], **kw)
    b = oracle.vtrace_probs(d["r"], d["v"], d["act"], d["logpi"][:, :T], taken, **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # A wrong layout of the taken entries is not the table form.
    assert not np.array_equal(_retrace_probs(dict(d, logmu=taken[:, ::-1].copy())),
                              _retrace_probs(d))
