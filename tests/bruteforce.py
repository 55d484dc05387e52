"""Forward-view (sum-form) definitions, written independently of the oracle.

The oracle computes each algorithm with a backward loop.  The functions here
compute the same quantities from the published *forward-view* sums, row by
row and step by step, in O(T^2) float64 (or exact ``Fraction``) arithmetic.
They share no code with ``oracle/`` and none with the HIP library.  They are
only fast enough for tiny inputs.

Notation (per row, t = 0..T-1): ``term_t``, ``trunc_t`` flags;
``done_t = term_t or trunc_t``; a truncation that is also a termination counts
as a termination; ``k_end(t)`` = first ``k >= t`` with ``done_k``, else
``T-1``; the successor value of step ``k`` is 0 after a termination, the
supplied ``trunc_values[k]`` after a truncation, ``V[k+1]`` otherwise
(``V[T]`` closes the window).
"""
import math


def _row(x, n):
    return None if x is None else x[n]


def _flags(term, trunc, n, T):
    te = [bool(term[n][t]) if term is not None else False for t in range(T)]
    tr = [bool(trunc[n][t]) if trunc is not None else False for t in range(T)]
    return te, tr


def _k_end(te, tr, t, T):
    for k in range(t, T):
        if te[k] or tr[k]:
            return k, True
    return T - 1, False


def _succ(v, tv, te, tr, k, T):
    """Successor value of step k (see module doc)."""
    if te[k]:
        return 0
    if tr[k]:
        return tv[k]
    return v[k + 1]


def returns(r, term, trunc, tv, bootstrap, gamma):
    """G_t = sum_{k=t}^{k_end} gamma^{k-t} r_k + gamma^{k_end-t+1} * tail, where
    tail = 0 (termination), tv (truncation) or the window bootstrap B."""
    N, T = len(r), len(r[0]) if len(r) else 0
    out = []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        B = bootstrap[n] if bootstrap is not None else 0
        row = []
        for t in range(T):
            k_end, cut = _k_end(te, tr, t, T)
            s = sum(gamma ** (k - t) * r[n][k] for k in range(t, k_end + 1))
            if cut:
                tail = 0 if te[k_end] else tv[n][k_end]
            else:
                tail = B
            row.append(s + gamma ** (k_end - t + 1) * tail)
        out.append(row)
    return out


def _deltas(r, v, tv, te, tr, T, gamma):
    return [r[k] + gamma * _succ(v, tv, te, tr, k, T) - v[k] for k in range(T)]


def gae(r, v, term, trunc, tv, gamma, lam):
    """A_t = sum_{k=t}^{k_end} (gamma*lam)^{k-t} delta_k   (Schulman et al. 2016)."""
    N, T = len(r), len(r[0]) if len(r) else 0
    adv = []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        d = _deltas(r[n], v[n], _row(tv, n), te, tr, T, gamma)
        row = []
        for t in range(T):
            k_end, _ = _k_end(te, tr, t, T)
            row.append(sum((gamma * lam) ** (k - t) * d[k] for k in range(t, k_end + 1)))
        adv.append(row)
    return adv


def td_lambda(r, v, term, trunc, tv, gamma, lam):
    """Forward-view lambda-return (Sutton & Barto, sec. 12.1), truncated at the
    episode end or the window end:
        G^lam_t = (1-lam) sum_{n=1}^{h-1} lam^{n-1} G^(n)_t + lam^{h-1} G^(h)_t,
    h = k_end - t + 1, G^(n)_t = sum_{i<n} gamma^i r_{t+i} + gamma^n W_n,
    W_n = V_{t+n} for n < h and W_h = successor value of step k_end."""
    N, T = len(r), len(r[0]) if len(r) else 0
    out = []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        rr, vv = r[n], v[n]
        row = []
        for t in range(T):
            k_end, _ = _k_end(te, tr, t, T)
            h = k_end - t + 1

            def G(m):
                s = sum(gamma ** i * rr[t + i] for i in range(m))
                W = vv[t + m] if m < h else _succ(vv, _row(tv, n), te, tr, k_end, T)
                return s + gamma ** m * W

            acc = (1 - lam) * sum(lam ** (m - 1) * G(m) for m in range(1, h))
            row.append(acc + lam ** (h - 1) * G(h))
        out.append(row)
    return out


def vtrace(r, v, log_rho, term, trunc, tv, gamma, lam, rho_bar, c_bar, pg_rho_bar):
    """IMPALA V-trace (Espeholt et al. 2018, eq. 1) with c_i = lam*min(c_bar, ratio_i):
        vs_t = V_t + sum_{k=t}^{k_end} gamma^{k-t} (prod_{i=t}^{k-1} c_i) rho_k delta_k,
    pg_t = min(pg_rho_bar, ratio_t) (r_t + gamma*nvs_t - V_t), nvs_t = 0 after a
    termination, tv_t after a truncation, vs_{t+1} otherwise (V_T at t = T-1)."""
    N, T = len(r), len(r[0]) if len(r) else 0
    vs_all, pg_all = [], []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        ratio = [math.exp(x) for x in log_rho[n]]
        rho = [min(rho_bar, x) for x in ratio]
        c = [lam * min(c_bar, x) for x in ratio]
        d = _deltas(r[n], v[n], _row(tv, n), te, tr, T, gamma)
        vs = []
        for t in range(T):
            k_end, _ = _k_end(te, tr, t, T)
            s = 0.0
            for k in range(t, k_end + 1):
                p = 1.0
                for i in range(t, k):
                    p *= c[i]
                s += gamma ** (k - t) * p * rho[k] * d[k]
            vs.append(v[n][t] + s)
        pg = []
        for t in range(T):
            if te[t]:
                nvs = 0.0
            elif tr[t]:
                nvs = tv[n][t]
            else:
                nvs = vs[t + 1] if t + 1 < T else v[n][T]
            pg.append(min(pg_rho_bar, ratio[t]) * (r[n][t] + gamma * nvs - v[n][t]))
        vs_all.append(vs)
        pg_all.append(pg)
    return vs_all, pg_all


def retrace(r, q, eq, log_rho, term, trunc, gamma, lam, c_bar):
    """Retrace(lambda) (Munos et al. 2016):
        Qret_t = Q_t + sum_{k=t}^{k_end} gamma^{k-t} (prod_{i=t+1}^{k} c_i)
                          (r_k + gamma*(1-term_k)*EQ_k - Q_k),
    c_i = lam * min(c_bar, ratio_i); EQ_k = E_pi Q(s_{k+1}, .)."""
    N, T = len(r), len(r[0]) if len(r) else 0
    out = []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        c = [lam * min(c_bar, math.exp(x)) for x in log_rho[n]]
        err = [r[n][k] + (0.0 if te[k] else gamma * eq[n][k]) - q[n][k] for k in range(T)]
        row = []
        for t in range(T):
            k_end, _ = _k_end(te, tr, t, T)
            s = 0.0
            for k in range(t, k_end + 1):
                p = 1.0
                for i in range(t + 1, k + 1):
                    p *= c[i]
                s += gamma ** (k - t) * p * err[k]
            row.append(q[n][t] + s)
        out.append(row)
    return out


def _episode_start(te, tr, t):
    """First step of the episode that contains step t (a boundary after step
    k-1 starts a new episode at k)."""
    s = t
    while s > 0 and not (te[s - 1] or tr[s - 1]):
        s -= 1
    return s


def eligibility_trace(x, term, trunc, z_init, decay):
    """z_t = sum_{k=s(t)}^{t} decay^{t-k} x_k (+ decay^{t+1} z_init if the episode
    of step t began before the window), s(t) = first step of t's episode."""
    N, T = len(x), len(x[0]) if len(x) else 0
    out = []
    for n in range(N):
        te, tr = _flags(term, trunc, n, T)
        z0 = z_init[n] if z_init is not None else 0
        row = []
        for t in range(T):
            s = _episode_start(te, tr, t)
            v = sum(decay ** (t - k) * x[n][k] for k in range(s, t + 1))
            if s == 0:
                v += decay ** (t + 1) * z0
            row.append(v)
        out.append(row)
    return out


def episodic_cumsum(x, term, trunc, s_init):
    """S_t = sum of x over the steps of t's episode up to t (+ s_init if that
    episode began before the window)."""
    return eligibility_trace(x, term, trunc, s_init, 1)


def affine_scan(alpha, beta, reset, carry, reverse):
    """Sum form of the segmented affine scan, row by row.

    Reverse:  A_t = sum_{k=t}^{T-1} (prod_{j=t}^{k-1} b_j) alpha_k
                    + (prod_{j=t}^{T-1} b_j) carry
    Forward:  A_t = sum_{k=0}^{t} (prod_{j=k+1}^{t} b_j) alpha_k
                    + (prod_{j=0}^{t} b_j) carry
    with b_j = 0 where reset_j is set, beta_j otherwise.  Every product is
    formed afresh for every (t, k): O(T^3), tiny inputs only.
    """
    out = []
    for n in range(len(alpha)):
        T = len(alpha[n])
        b = [0 if (reset is not None and reset[n][j]) else beta[n][j] for j in range(T)]
        c = 0 if carry is None else carry[n]
        row = []
        for t in range(T):
            ks = range(t, T) if reverse else range(0, t + 1)
            total = 0
            for k in ks:
                js = range(t, k) if reverse else range(k + 1, t + 1)
                total += math.prod(b[j] for j in js) * alpha[n][k]
            js = range(t, T) if reverse else range(0, t + 1)
            total += math.prod(b[j] for j in js) * c
            row.append(total)
        out.append(row)
    return out
