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
 * Every function returns 0 on success and -1 on a NULL required pointer or a
 * negative size.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define AT(p, n, t, ld) ((p)[(size_t)(n) * (size_t)(ld) + (size_t)(t)])

static int flag_at(const uint8_t *f, int64_t n, int64_t t, int64_t T)
{
    return f != NULL && AT(f, n, t, T) != 0;
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
 * Here the window bootstrap lives in the carry A_T (Method 3, rollout windows).
 */
int oracle_returns(int64_t N, int64_t T, const double *r, const uint8_t *term,
                   const uint8_t *trunc, const double *tv, const double *bootstrap,
                   double gamma, double *G)
{
    if (N < 0 || T < 0 || (N > 0 && T > 0 && (r == NULL || G == NULL)) ||
        (trunc != NULL && tv == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double g = bootstrap != NULL ? bootstrap[n] : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double succ;
            if (flag_at(term, n, t, T))
                succ = 0.0;
            else if (flag_at(trunc, n, t, T))
                succ = AT(tv, n, t, T);
            else
                succ = g;
            g = AT(r, n, t, T) + gamma * succ;
            AT(G, n, t, T) = g;
        }
    }
    return 0;
}

/*
 * Generalized advantage estimation (Schulman et al. 2016), cut at episode
 * ends (rl-triton, Method 1 "GAE"; Method 3):
 *   delta_t = r_t + gamma * next_value_t - V_t
 *   A_t     = delta_t + gamma*lam * A_{t+1}    if not done_t
 *   A_t     = delta_t                          if done_t
 *   A_T     = 0: the window bootstrap V_T enters through delta_{T-1}.
 *   targets_t = A_t + V_t.
 */
int oracle_gae(int64_t N, int64_t T, const double *r, const double *v,
               const uint8_t *term, const uint8_t *trunc, const double *tv,
               double gamma, double lam, double *adv, double *targets)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || adv == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double a = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double vt = AT(v, n, t, T + 1);
            double delta = AT(r, n, t, T) + gamma * next_value(v, tv, term, trunc, n, t, T) - vt;
            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
            a = done ? delta : delta + gamma * lam * a;
            AT(adv, n, t, T) = a;
            if (targets != NULL)
                AT(targets, n, t, T) = a + vt;
        }
    }
    return 0;
}

/*
 * TD(lambda) returns (rl-triton, Method 1 "TD(lambda) returns"), backward
 * (recursive) lambda-return of Sutton & Barto with episode cuts:
 *   G_t = r_t + gamma * next_value_t                                if done_t
 *   G_t = r_t + gamma * ((1 - lam) * V_{t+1} + lam * G_{t+1})       otherwise
 *   G_T = V_T (the window bootstrap; equivalently (1-lam)V_T + lam V_T).
 * This form is independent of the GAE function above; the two agree as
 * G_t = A_t + V_t only in exact arithmetic.
 */
int oracle_td_lambda(int64_t N, int64_t T, const double *r, const double *v,
                     const uint8_t *term, const uint8_t *trunc, const double *tv,
                     double gamma, double lam, double *ret)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || ret == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double g = AT(v, n, T, T + 1);
        for (int64_t t = T - 1; t >= 0; --t) {
            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
            double rt = AT(r, n, t, T);
            if (done)
                g = rt + gamma * next_value(v, tv, term, trunc, n, t, T);
            else
                g = rt + gamma * ((1.0 - lam) * AT(v, n, t + 1, T + 1) + lam * g);
            AT(ret, n, t, T) = g;
        }
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
 *   v_T    = V_T (window end: the correction beyond the window is zero).
 *   pg_t   = min(pg_rho_bar, exp(log_rho_t)) * (r_t + gamma * nv_t - V_t),
 *            nv_t = 0 if term_t, tv_t if a truncation, v_{t+1} otherwise.
 * pg may be NULL.
 */
int oracle_vtrace(int64_t N, int64_t T, const double *r, const double *v,
                  const double *log_rho, const uint8_t *term, const uint8_t *trunc,
                  const double *tv, double gamma, double lam, double rho_bar,
                  double c_bar, double pg_rho_bar, double *vs, double *pg)
{
    if (N < 0 || T < 0 || (trunc != NULL && tv == NULL))
        return -1;
    if (N > 0 && T > 0 && (r == NULL || v == NULL || log_rho == NULL || vs == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double v_next = AT(v, n, T, T + 1); /* v_{t+1}, starting with v_T = V_T */
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
            if (!done)
                vs_t += gamma * c * (v_next - AT(v, n, t + 1, T + 1));
            if (pg != NULL) {
                double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : v_next);
                AT(pg, n, t, T) = fmin(pg_rho_bar, ratio) * (rt + gamma * nvs - vt);
            }
            AT(vs, n, t, T) = vs_t;
            v_next = vs_t;
        }
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
 * cut; at a termination EQ_t is dropped.  At t = T-1 the correction term is
 * absent because c_T and Q_T lie outside the window: EQ_{T-1} is the window
 * bootstrap, in alpha_{T-1} (Method 3, rollout windows).
 */
int oracle_retrace(int64_t N, int64_t T, const double *r, const double *q,
                   const double *eq, const double *log_rho, const uint8_t *term,
                   const uint8_t *trunc, double gamma, double lam, double c_bar,
                   double *qret)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (r == NULL || q == NULL || eq == NULL || log_rho == NULL || qret == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double qret_next = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int term_t = flag_at(term, n, t, T);
            int done = term_t || flag_at(trunc, n, t, T);
            double target = AT(r, n, t, T) + (term_t ? 0.0 : gamma * AT(eq, n, t, T));
            if (!done && t < T - 1) {
                double c_next = lam * fmin(c_bar, exp(AT(log_rho, n, t + 1, T)));
                target += gamma * c_next * (qret_next - AT(q, n, t + 1, T));
            }
            AT(qret, n, t, T) = target;
            qret_next = target;
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
 * used as given (the caller zeroes it if the previous window ended an
 * episode).
 */

/* Accumulating eligibility trace:
 *   z_t = x_t + gamma*lam * z_{t-1}   if not done_{t-1},
 *   z_t = x_t                         if done_{t-1};   z_{-1} = z_init. */
int oracle_eligibility_trace(int64_t N, int64_t T, const double *x, const uint8_t *term,
                             const uint8_t *trunc, const double *z_init, double gamma,
                             double lam, double *z)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (x == NULL || z == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double prev = z_init != NULL ? z_init[n] : 0.0;
        int prev_done = 0;
        for (int64_t t = 0; t < T; ++t) {
            double zt = AT(x, n, t, T) + (prev_done ? 0.0 : gamma * lam * prev);
            AT(z, n, t, T) = zt;
            prev = zt;
            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
        }
    }
    return 0;
}

/* Episodic prefix sum:
 *   S_t = x_t + S_{t-1}   if not done_{t-1},
 *   S_t = x_t             if done_{t-1};   S_{-1} = s_init. */
int oracle_episodic_cumsum(int64_t N, int64_t T, const double *x, const uint8_t *term,
                           const uint8_t *trunc, const double *s_init, double *s)
{
    if (N < 0 || T < 0)
        return -1;
    if (N > 0 && T > 0 && (x == NULL || s == NULL))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double prev = s_init != NULL ? s_init[n] : 0.0;
        int prev_done = 0;
        for (int64_t t = 0; t < T; ++t) {
            double st = AT(x, n, t, T) + (prev_done ? 0.0 : prev);
            AT(s, n, t, T) = st;
            prev = st;
            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);
        }
    }
    return 0;
}
