/*
 * oracle.c -- fp64 CPU oracle for reverse-time credit-assignment recurrences.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code.
 *
 * Source of truth.  "rl-triton" below means the explainer pages of
 * "rl-triton: High-Performance Triton GPU Kernels for Reinforcement Learning
 * Credit Assignment" (Zehnder, 2026).  Their Technical summary states:
 *   - Method 1 (unified algebraic framework): every algorithm here is an
 *     instance of the reverse-time first-order recurrence
 *         A_t = alpha_t + beta_t * A_{t+1}                         (eq. R)
 *   - Method 3 (explicit boundary semantics):
 *       * a natural episode end (termination) makes the successor value zero,
 *         a truncation uses a supplied bootstrap value;
 *       * at the end of the rollout window (t = T-1) the bootstrap enters
 *         either the local term alpha_{T-1} or the scan carry A_T, never both.
 * The pages do not print the per-algorithm coefficients.  Each function below
 * writes out the standard published definition of its algorithm in its
 * recursive (backward) form; the coefficient choice is noted per function.
 *
 * Form.  One plain backward loop t = T-1 ... 0 per row, in double precision,
 * on contiguous row-major inputs.  No blocking, no reordering, no scan.
 *
 * Shared notation, per row, t = 0 .. T-1:
 *   term_t  = terminated[t] != 0            (NULL array: never)
 *   trunc_t = truncated[t]  != 0            (NULL array: never)
 *   done_t  = term_t || trunc_t             the episode ends after step t
 *   boot_t  = trunc_t && !term_t            truncation that is not also a
 *                                           termination (termination wins)
 *   next value after step t:
 *       0                 if term_t
 *       tv_t              if boot_t   (value of the true final observation)
 *       V_{t+1}           otherwise   (V has T+1 columns; V_T closes the window)
 *
 * Window carries (rl-triton, Method 3 "rollout windows"; Method 1: the
 * operator is associative, so a rollout may be cut along time).  A rollout
 * longer than one window is processed as consecutive windows.  Per row:
 *   carry_in   the scan state just past the window end (reverse recurrences)
 *              or just before its start (forward ones), in the units each
 *              function states; NULL means 0, the plain windowed result.
 *              (returns: the bootstrap; forward mirrors: the initial value.)
 *   carry_out  [N], NULL = not wanted: the value the neighbouring window
 *              (the earlier one for reverse recurrences, the later one for
 *              forward ones) takes as its carry_in, so that consecutive
 *              windows reproduce the result of one long window.
 *   map_out    [N, 2], NULL = not wanted: (a, b) with
 *              carry_out = a + b * carry_in for every carry_in.  a is
 *              carry_out computed from carry 0 (a second copy of the state,
 *              suffix 0, run from 0 beside the real one); b is its derivative
 *              with respect to carry_in (forward-mode differentiation of the
 *              same loop: a variable prefixed d, updated beside the state).
 *              Windows evaluated independently chain through these maps.
 *
 * Every function returns 0 on success and -1 on a NULL required pointer or a
 * negative size.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define AT(p, n, t, ld) ((p)[(size_t)(n) * (size_t)(ld) + (size_t)(t)])

static int flag_at(const uint8_t *f, int64_t n, int64_t t, int64_t T)
{
    return f != NULL && AT(f, n, t, T) != 0;
}

/* Store the carry and the carry map of row n (either pointer may be NULL). */
static void put_carry(double *carry_out, double *map_out, int64_t n, double carry,
                      double a, double b)
{
    if (carry_out != NULL)
        carry_out[n] = carry;
    if (map_out != NULL) {
        map_out[2 * n] = a;
        map_out[2 * n + 1] = b;
    }
}

/* Successor value of step t (see the header).  v is [N, T+1]. */
static double next_value(const double *v, const double *tv, const uint8_t *term,
                         const uint8_t *trunc, int64_t n, int64_t t, int64_t T)
{
    if (flag_at(term, n, t, T))
        return 0.0;
    if (flag_at(trunc, n, t, T))
        return AT(tv, n, t, T);
    return AT(v, n, t + 1, T + 1);
}

/*
 * Discounted returns (rl-triton, Method 1: "discounted returns").
 *   G_t = r_t + gamma * G_{t+1}    inside an episode,
 *   G_t = r_t                      after a termination,
 *   G_t = r_t + gamma * tv_t       after a truncation,
 *   G_T = B                        per-row window bootstrap (NULL: 0).
 * Here the window bootstrap lives in the carry A_T (Method 3, rollout windows):
 * carry_in is B, carry_out is G_0.
 */
int oracle_returns(int64_t N, int64_t T, const double *r, const uint8_t *term,
                   const uint8_t *trunc, const double *tv, const double *bootstrap,
                   double gamma, double *G, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || (N > 0 && T > 0 && (r == NULL || G == NULL)) ||
        (trunc != NULL && tv == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double g = bootstrap != NULL ? bootstrap[n] : 0.0;
        double g0 = 0.0, dg = 1.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double succ, succ0, dsucc;
            if (flag_at(term, n, t, T)) {
                succ = succ0 = dsucc = 0.0;
            } else if (flag_at(trunc, n, t, T)) {
                succ = succ0 = AT(tv, n, t, T);
                dsucc = 0.0;
            } else {
                succ = g;
                succ0 = g0;
                dsucc = dg;
            }
            g = AT(r, n, t, T) + gamma * succ;
            g0 = AT(r, n, t, T) + gamma * succ0;
            dg = gamma * dsucc;
            AT(G, n, t, T) = g;
        }
        put_carry(carry_out, map_out, n, g, g0, dg);
    }
    return 0;
}

/*
 * Generalized advantage estimation (Schulman et al. 2016), cut at episode
 * ends (rl-triton, Method 1 "GAE"; Method 3):
 *   delta_t = r_t + gamma * next_value_t - V_t
 *   A_t     = delta_t + gamma*lam * A_{t+1}    if not done_t
 *   A_t     = delta_t                          if done_t
 *   A_T     = carry_in (NULL: 0): the window bootstrap V_T enters through
 *             delta_{T-1}; carry_in is the advantage A_T of the step after
 *             the window, and carry_out is A_0.
 *   targets_t = A_t + V_t.
 */
int oracle_gae(int64_t N, int64_t T, const double *r, const double *v,
               const uint8_t *term, const uint8_t *trunc, const double *tv,
               double gamma, double lam, double *adv, double *targets,
               const double *carry_in, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || adv == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double a = carry_in != NULL ? carry_in[n] : 0.0;
        double a0 = 0.0, da = 1.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double vt = AT(v, n, t, T + 1);
            double delta = AT(r, n, t, T) + gamma * next_value(v, tv, term, trunc, n, t, T) - vt;
            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
            a = done ? delta : delta + gamma * lam * a;
            a0 = done ? delta : delta + gamma * lam * a0;
            da = done ? 0.0 : gamma * lam * da;
            AT(adv, n, t, T) = a;
            if (targets != NULL)
                AT(targets, n, t, T) = a + vt;
        }
        put_carry(carry_out, map_out, n, a, a0, da);
    }
    return 0;
}

/*
 * TD(lambda) returns (rl-triton, Method 1 "TD(lambda) returns"), backward
 * (recursive) lambda-return of Sutton & Barto with episode cuts:
 *   G_t = r_t + gamma * next_value_t                                if done_t
 *   G_t = r_t + gamma * ((1 - lam) * V_{t+1} + lam * G_{t+1})       otherwise
 *   G_T = V_T + carry_in (the window bootstrap, plus the lambda-return
 *         excess G_T - V_T of the step after the window; NULL: 0).
 * carry_out is G_0 - V_0.  This form is independent of the GAE function
 * above; the two agree as G_t = A_t + V_t only in exact arithmetic.
 */
int oracle_td_lambda(int64_t N, int64_t T, const double *r, const double *v,
                     const uint8_t *term, const uint8_t *trunc, const double *tv,
                     double gamma, double lam, double *ret,
                     const double *carry_in, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || ret == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double g = AT(v, n, T, T + 1) + (carry_in != NULL ? carry_in[n] : 0.0);
        double g0 = AT(v, n, T, T + 1), dg = 1.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
            double rt = AT(r, n, t, T);
            if (done) {
                g = rt + gamma * next_value(v, tv, term, trunc, n, t, T);
                g0 = g;
                dg = 0.0;
            } else {
                g = rt + gamma * ((1.0 - lam) * AT(v, n, t + 1, T + 1) + lam * g);
                g0 = rt + gamma * ((1.0 - lam) * AT(v, n, t + 1, T + 1) + lam * g0);
                dg = gamma * lam * dg;
            }
            AT(ret, n, t, T) = g;
        }
        double v0 = AT(v, n, 0, T + 1);
        put_carry(carry_out, map_out, n, g - v0, g0 - v0, dg);
    }
    return 0;
}

/*
 * V-trace (Espeholt et al. 2018, IMPALA, eq. 1 in its recursive form), with
 * the lambda-scaled trace (rl-triton, Method 1 "V-trace"):
 *   rho_t  = min(rho_bar, exp(log_rho_t))
 *   c_t    = lam * min(c_bar, exp(log_rho_t))
 *   v_t    = V_t + rho_t * (r_t + gamma * next_value_t - V_t)
 *                + gamma * c_t * (v_{t+1} - V_{t+1})      (the last term only
 *                                                          if not done_t)
 *   v_T    = V_T + carry_in (window end: the correction v_T - V_T beyond
 *            the window, zero when carry_in is NULL).
 *   pg_t   = min(pg_rho_bar, exp(log_rho_t)) * (r_t + gamma * nv_t - V_t),
 *            nv_t = 0 if term_t, tv_t if a truncation, v_{t+1} otherwise.
 * pg may be NULL.  carry_out is v_0 - V_0.
 */
int oracle_vtrace(int64_t N, int64_t T, const double *r, const double *v,
                  const double *log_rho, const uint8_t *term, const uint8_t *trunc,
                  const double *tv, double gamma, double lam, double rho_bar,
                  double c_bar, double pg_rho_bar, double *vs, double *pg,
                  const double *carry_in, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || log_rho == NULL || vs == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        /* v_{t+1}, starting with v_T */
        double v_next = AT(v, n, T, T + 1) + (carry_in != NULL ? carry_in[n] : 0.0);
        double v_next0 = AT(v, n, T, T + 1), dv_next = 1.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double ratio = exp(AT(log_rho, n, t, T));
            double rho = fmin(rho_bar, ratio);
            double c = lam * fmin(c_bar, ratio);
            double vt = AT(v, n, t, T + 1);
            double rt = AT(r, n, t, T);
            int term_t = flag_at(term, n, t, T);
            int done = term_t || flag_at(trunc, n, t, T);
            double nv = next_value(v, tv, term, trunc, n, t, T);
            double vs_t = vt + rho * (rt + gamma * nv - vt);
            double vs0_t = vs_t, dvs_t = 0.0;
            if (!done) {
                vs_t += gamma * c * (v_next - AT(v, n, t + 1, T + 1));
                vs0_t += gamma * c * (v_next0 - AT(v, n, t + 1, T + 1));
                dvs_t = gamma * c * dv_next;
            }
            if (pg != NULL) {
                double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : v_next);
                AT(pg, n, t, T) = fmin(pg_rho_bar, ratio) * (rt + gamma * nvs - vt);
            }
            AT(vs, n, t, T) = vs_t;
            v_next = vs_t;
            v_next0 = vs0_t;
            dv_next = dvs_t;
        }
        double v0 = AT(v, n, 0, T + 1);
        put_carry(carry_out, map_out, n, v_next - v0, v_next0 - v0, dv_next);
    }
    return 0;
}

/*
 * Retrace(lambda) (Munos et al. 2016) in its recursive form
 * (rl-triton, Method 1 "Retrace(lambda)"):
 *   c_t    = lam * min(c_bar, exp(log_rho_t))
 *   Qret_t = r_t + gamma * (1 - term_t) * EQ_t
 *            + gamma * c_{t+1} * (Qret_{t+1} - Q_{t+1})    (only if not done_t
 *                                                           and t < T-1)
 * where Q_t = Q(s_t, a_t) and EQ_t = E_pi Q(s_{t+1}, .).  At a truncation the
 * supplied EQ_t (value of the true final state) is kept and only the trace is
 * cut; at a termination EQ_t is dropped.  At t = T-1 the correction
 * c_T * (Qret_T - Q_T) involves the step after the window: it is carry_in
 * (NULL: 0, the plain window, where EQ_{T-1} is the window bootstrap, in
 * alpha_{T-1}; Method 3, rollout windows).  carry_out is the same quantity
 * for the window's first step, c_0 * (Qret_0 - Q_0).
 */
int oracle_retrace(int64_t N, int64_t T, const double *r, const double *q,
                   const double *eq, const double *log_rho, const uint8_t *term,
                   const uint8_t *trunc, double gamma, double lam, double c_bar,
                   double *qret, const double *carry_in, double *carry_out,
                   double *map_out)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (r == NULL || q == NULL || eq == NULL || log_rho == NULL || qret == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double qret_next = 0.0, qret_next0 = 0.0, dqret_next = 0.0;
        double carry = carry_in != NULL ? carry_in[n] : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int term_t = flag_at(term, n, t, T);
            int done = term_t || flag_at(trunc, n, t, T);
            double target = AT(r, n, t, T) + (term_t ? 0.0 : gamma * AT(eq, n, t, T));
            double target0 = target, dtarget = 0.0;
            if (!done && t < T - 1) {
                double c_next = lam * fmin(c_bar, exp(AT(log_rho, n, t + 1, T)));
                target += gamma * c_next * (qret_next - AT(q, n, t + 1, T));
                target0 += gamma * c_next * (qret_next0 - AT(q, n, t + 1, T));
                dtarget = gamma * c_next * dqret_next;
            } else if (!done) { /* t = T-1: the correction from the step after the window */
                target += gamma * carry;
                dtarget = gamma;
            }
            AT(qret, n, t, T) = target;
            qret_next = target;
            qret_next0 = target0;
            dqret_next = dtarget;
        }
        if (T > 0) {
            double c0 = lam * fmin(c_bar, exp(AT(log_rho, n, 0, T)));
            double q0 = AT(q, n, 0, T);
            put_carry(carry_out, map_out, n, c0 * (qret_next - q0), c0 * (qret_next0 - q0),
                      c0 * dqret_next);
        } else {
            put_carry(carry_out, map_out, n, carry, 0.0, 1.0);
        }
    }
    return 0;
}

/*
 * Forward-time recurrences (rl-triton, Method 1: eligibility traces and
 * episodic prefix sums are the forward-time mirror of eq. R):
 *     A_t = alpha_t + beta_t * A_{t-1},   t = 0 .. T-1.
 * An episode boundary after step t-1 (done_{t-1}) restarts the recurrence at
 * step t.  A_{-1} is a per-row carry from before the window (NULL: 0); it is
 * used as given.  carry_out is what the next window's first step receives:
 * A_{T-1}, or 0 if the episode ends after step T-1 (done_{T-1}).
 */

/* Accumulating eligibility trace:
 *   z_t = x_t + gamma*lam * z_{t-1}   if not done_{t-1},
 *   z_t = x_t                         if done_{t-1};   z_{-1} = z_init. */
int oracle_eligibility_trace(int64_t N, int64_t T, const double *x, const uint8_t *term,
                             const uint8_t *trunc, const double *z_init, double gamma,
                             double lam, double *z, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (x == NULL || z == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double prev = z_init != NULL ? z_init[n] : 0.0;
        double prev0 = 0.0, dprev = 1.0;
        int prev_done = 0;
        for (int64_t t = 0; t < T; ++t) {
            double z0t = AT(x, n, t, T) + (prev_done ? 0.0 : gamma * lam * prev0);
            double dzt = prev_done ? 0.0 : gamma * lam * dprev;
            prev0 = z0t;
            dprev = dzt;
            double zt = AT(x, n, t, T) + (prev_done ? 0.0 : gamma * lam * prev);
            AT(z, n, t, T) = zt;
            prev = zt;
            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
        }
        if (prev_done)
            put_carry(carry_out, map_out, n, 0.0, 0.0, 0.0);
        else
            put_carry(carry_out, map_out, n, prev, prev0, dprev);
    }
    return 0;
}

/* Episodic prefix sum:
 *   S_t = x_t + S_{t-1}   if not done_{t-1},
 *   S_t = x_t             if done_{t-1};   S_{-1} = s_init. */
int oracle_episodic_cumsum(int64_t N, int64_t T, const double *x, const uint8_t *term,
                           const uint8_t *trunc, const double *s_init, double *s,
                           double *carry_out, double *map_out)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (x == NULL || s == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double prev = s_init != NULL ? s_init[n] : 0.0;
        double prev0 = 0.0, dprev = 1.0;
        int prev_done = 0;
        for (int64_t t = 0; t < T; ++t) {
            double s0t = AT(x, n, t, T) + (prev_done ? 0.0 : prev0);
            double dst = prev_done ? 0.0 : dprev;
            prev0 = s0t;
            dprev = dst;
            double st = AT(x, n, t, T) + (prev_done ? 0.0 : prev);
            AT(s, n, t, T) = st;
            prev = st;
            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
        }
        double keep = prev_done ? 0.0 : 1.0; /* nothing crosses an episode end */
        put_carry(carry_out, map_out, n, keep * prev, keep * prev0, keep * dprev);
    }
    return 0;
}

/*
 * Generic segmented affine scan (rl-triton, Method 1: eq. R with arbitrary
 * coefficient sequences, of which every algorithm above is an instance).
 *   reverse != 0:  A_t = alpha_t + beta'_t * A_{t+1},  t = T-1 .. 0,  A_T = carry_in
 *   reverse == 0:  A_t = alpha_t + beta'_t * A_{t-1},  t = 0 .. T-1,  A_{-1} = carry_in
 * with beta'_t = 0 where reset_t is set (step t starts a segment: nothing
 * flows into it from its neighbour) and beta_t elsewhere; reset NULL: never.
 * carry_in NULL: 0.  carry_out is the last state computed: A_0 (reverse) or
 * A_{T-1} (forward); a reset in the next window is that window's own flag.
 */
int oracle_affine_scan(int64_t N, int64_t T, const double *alpha, const double *beta,
                       const uint8_t *reset, int reverse, const double *carry_in,
                       double *out, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (alpha == NULL || beta == NULL || out == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double a = carry_in != NULL ? carry_in[n] : 0.0;
        double a0 = 0.0, da = 1.0;
        for (int64_t i = 0; i < T; ++i) {
            int64_t t = reverse ? T - 1 - i : i;
            double b = flag_at(reset, n, t, T) ? 0.0 : AT(beta, n, t, T);
            a = AT(alpha, n, t, T) + b * a;
            a0 = AT(alpha, n, t, T) + b * a0;
            da = b * da;
            AT(out, n, t, T) = a;
        }
        put_carry(carry_out, map_out, n, a, a0, da);
    }
    return 0;
}

/*
 * Retrace(lambda) and V-trace from the policies' log-probability tables
 * (rl-triton, Results: the heavier Retrace workload loads the action
 * probabilities at every step).  Per row, with A actions and a_t the action
 * taken at step t (0 <= a_t < A):
 *   log_rho_t = log_pi[t][a_t] - log_mu[t][a_t]      target over behaviour
 * Retrace also reads action values and the target policy one step ahead:
 *   q       [N, T+1, A]   Q(s_t, a); slice T is the state after the window
 *   log_pi  [N, T+1, A]   log pi(a | s_t); slice T likewise
 *   q_taken_t = q[t][a_t]
 *   EQ_t      = sum over a of exp(log_pi[t+1][a]) * q[t+1][a]   (E_pi Q(s_{t+1}, .))
 *   except after a truncation that is not a termination, where s_{t+1} in the
 *   tables is the next episode's first state: EQ_t = trunc_eq[t], the same
 *   expectation at the true final state, supplied by the caller.
 * V-trace reads log_pi [N, T, A] (no slice T).  log_mu is [N, T, A] for both,
 * or, with mu_taken != 0, [N, T] holding log mu(a_t | s_t) of the taken
 * actions only.  With these [N, T] quantities the result is that of
 * oracle_retrace / oracle_vtrace above (window carries passed through).  An
 * action outside [0, A) is rejected (-1).
 */
static int derive_probs(int64_t N, int64_t T, int64_t A, int pi_slices, const int32_t *actions,
                        const double *log_pi, const double *log_mu, int mu_taken,
                        double *log_rho)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < T; ++t) {
            int32_t a = actions[n * T + t];
            if (a < 0 || a >= A)
                return -1;
            double lp = log_pi[((size_t)n * (size_t)(T + pi_slices) + (size_t)t) * (size_t)A + (size_t)a];
            double lm = mu_taken ? log_mu[n * T + t]
                                 : log_mu[((size_t)n * (size_t)T + (size_t)t) * (size_t)A + (size_t)a];
            log_rho[n * T + t] = lp - lm;
        }
    return 0;
}

int oracle_retrace_probs(int64_t N, int64_t T, int64_t A, const double *r, const double *q,
                         const int32_t *actions, const double *log_pi, const double *log_mu,
                         int mu_taken, const uint8_t *term, const uint8_t *trunc,
                         const double *trunc_eq,
                         double gamma, double lam, double c_bar, double *qret,
                         const double *carry_in, double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || A < 1 || (trunc != NULL && trunc_eq == NULL))
        return -1;
    if (N == 0 || T == 0)
        return oracle_retrace(N, T, r, NULL, NULL, NULL, term, trunc, gamma, lam, c_bar, qret,
                              carry_in, carry_out, map_out);
    if (r == NULL || q == NULL || actions == NULL || log_pi == NULL || log_mu == NULL ||
        qret == NULL)
        return -1;
    size_t nt = (size_t)N * (size_t)T;
    double *q_taken = malloc(nt * sizeof(double));
    double *eq = malloc(nt * sizeof(double));
    double *log_rho = malloc(nt * sizeof(double));
    int rc = -1;
    if (q_taken == NULL || eq == NULL || log_rho == NULL)
        goto out;
    if (derive_probs(N, T, A, 1, actions, log_pi, log_mu, mu_taken, log_rho) != 0)
        goto out;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < T; ++t) {
            size_t here = ((size_t)n * (size_t)(T + 1) + (size_t)t) * (size_t)A;
            size_t next = here + (size_t)A;
            q_taken[n * T + t] = q[here + (size_t)actions[n * T + t]];
            if (flag_at(trunc, n, t, T) && !flag_at(term, n, t, T)) {
                eq[n * T + t] = AT(trunc_eq, n, t, T);
            } else {
                double e = 0.0;
                for (int64_t b = 0; b < A; ++b)
                    e += exp(log_pi[next + (size_t)b]) * q[next + (size_t)b];
                eq[n * T + t] = e;
            }
        }
    rc = oracle_retrace(N, T, r, q_taken, eq, log_rho, term, trunc, gamma, lam, c_bar, qret,
                        carry_in, carry_out, map_out);
out:
    free(q_taken);
    free(eq);
    free(log_rho);
    return rc;
}

int oracle_vtrace_probs(int64_t N, int64_t T, int64_t A, const double *r, const double *v,
                        const int32_t *actions, const double *log_pi, const double *log_mu,
                        int mu_taken, const uint8_t *term, const uint8_t *trunc,
                        const double *tv,
                        double gamma, double lam, double rho_bar, double c_bar,
                        double pg_rho_bar, double *vs, double *pg, const double *carry_in,
                        double *carry_out, double *map_out)
{
    if (N < 0 || T < 0 || A < 1 || (trunc != NULL && tv == NULL))
        return -1;
    if (N == 0 || T == 0)
        return oracle_vtrace(N, T, r, v, NULL, term, trunc, tv, gamma, lam, rho_bar, c_bar,
                             pg_rho_bar, vs, pg, carry_in, carry_out, map_out);
    if (r == NULL || v == NULL || actions == NULL || log_pi == NULL || log_mu == NULL ||
        vs == NULL)
        return -1;
    double *log_rho = malloc((size_t)N * (size_t)T * sizeof(double));
    int rc = -1;
    if (log_rho != NULL && derive_probs(N, T, A, 0, actions, log_pi, log_mu, mu_taken, log_rho) == 0)
        rc = oracle_vtrace(N, T, r, v, log_rho, term, trunc, tv, gamma, lam, rho_bar, c_bar,
                           pg_rho_bar, vs, pg, carry_in, carry_out, map_out);
    free(log_rho);
    return rc;
}
