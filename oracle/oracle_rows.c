/*
 * oracle_rows.c -- the fp64 oracle of oracle.c on several host threads.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c: it times the oracle on every host
 * core for the benchmark's CPU baseline.  Rows are independent (every
 * recurrence runs along one row), so each driver cuts the N rows into
 * `nthreads` contiguous slices and hands each slice, with every array
 * pointer moved to its first row, to the unchanged serial function of
 * oracle.c on its own OpenMP thread.  No arithmetic lives here.
 *
 * Arrays are row-major and contiguous, as oracle.c takes them: [N, T]
 * (values [N, T+1]; policy tables [N, S, A]).  Returns 0, or -1 if any slice
 * was rejected (the serial function's own argument checks).
 */
#include <stddef.h>
#include <stdint.h>

#include <omp.h>

int oracle_returns(int64_t N, int64_t T, const double *r, const uint8_t *term,
                   const uint8_t *trunc, const double *tv, const double *bootstrap,
                   double gamma, double *G, double *carry_out, double *map_out);
int oracle_gae(int64_t N, int64_t T, const double *r, const double *v,
               const uint8_t *term, const uint8_t *trunc, const double *tv,
               double gamma, double lam, double *adv, double *targets,
               const double *carry_in, double *carry_out, double *map_out);
int oracle_td_lambda(int64_t N, int64_t T, const double *r, const double *v,
                     const uint8_t *term, const uint8_t *trunc, const double *tv,
                     double gamma, double lam, double *ret,
                     const double *carry_in, double *carry_out, double *map_out);
int oracle_vtrace(int64_t N, int64_t T, const double *r, const double *v,
                  const double *log_rho, const uint8_t *term, const uint8_t *trunc,
                  const double *tv, double gamma, double lam, double rho_bar,
                  double c_bar, double pg_rho_bar, double *vs, double *pg,
                  const double *carry_in, double *carry_out, double *map_out);
int oracle_retrace(int64_t N, int64_t T, const double *r, const double *q,
                   const double *eq, const double *log_rho, const uint8_t *term,
                   const uint8_t *trunc, double gamma, double lam, double c_bar,
                   double *qret, const double *carry_in, double *carry_out,
                   double *map_out);
int oracle_eligibility_trace(int64_t N, int64_t T, const double *x, const uint8_t *term,
                             const uint8_t *trunc, const double *z_init, double gamma,
                             double lam, double *z, double *carry_out, double *map_out);
int oracle_episodic_cumsum(int64_t N, int64_t T, const double *x, const uint8_t *term,
                           const uint8_t *trunc, const double *s_init, double *s,
                           double *carry_out, double *map_out);
int oracle_retrace_probs(int64_t N, int64_t T, int64_t A, const double *r, const double *q,
                         const int32_t *actions, const double *log_pi, const double *log_mu,
                         int mu_taken, const uint8_t *term, const uint8_t *trunc,
                         const double *trunc_eq,
                         double gamma, double lam, double c_bar, double *qret,
                         const double *carry_in, double *carry_out, double *map_out);
int oracle_vtrace_probs(int64_t N, int64_t T, int64_t A, const double *r, const double *v,
                        const int32_t *actions, const double *log_pi, const double *log_mu,
                        int mu_taken, const uint8_t *term, const uint8_t *trunc,
                        const double *tv,
                        double gamma, double lam, double rho_bar, double c_bar,
                        double pg_rho_bar, double *vs, double *pg, const double *carry_in,
                        double *carry_out, double *map_out);

/* Row n0 of a row-major array of row length ld (NULL stays NULL). */
#define ROW(p, n0, ld) ((p) != NULL ? (p) + (size_t)(n0) * (size_t)(ld) : NULL)

/* Run BODY once per slice [n0, n0 + n) of the N rows, nthreads slices, one
 * per OpenMP thread; BODY sets rc_ if its slice was rejected, and the
 * driver returns -1 if any was. */
#define FOR_SLICES(N, nthreads, BODY)                                            \
    int slices_ = (nthreads) < 1 ? 1 : (nthreads);                               \
    int rc_ = 0;                                                                 \
    _Pragma("omp parallel for num_threads(slices_) schedule(static, 1) reduction(|:rc_)") \
    for (int k_ = 0; k_ < slices_; ++k_) {                                       \
        int64_t n0 = (N) * k_ / slices_;                                         \
        int64_t n = (N) * (k_ + 1) / slices_ - n0;                               \
        BODY                                                                     \
    }                                                                            \
    return rc_ ? -1 : 0

int oracle_rows_threads(void) { return omp_get_max_threads(); }

int oracle_rows_returns(int nthreads, int64_t N, int64_t T, const double *r,
                        const uint8_t *term, const uint8_t *trunc, const double *tv,
                        const double *bootstrap, double gamma, double *G)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_returns(n, T, ROW(r, n0, T), ROW(term, n0, T), ROW(trunc, n0, T),
                              ROW(tv, n0, T), ROW(bootstrap, n0, 1), gamma, ROW(G, n0, T),
                              NULL, NULL) != 0;
    });
}

int oracle_rows_gae(int nthreads, int64_t N, int64_t T, const double *r, const double *v,
                    const uint8_t *term, const uint8_t *trunc, const double *tv,
                    double gamma, double lam, double *adv, double *targets)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_gae(n, T, ROW(r, n0, T), ROW(v, n0, T + 1), ROW(term, n0, T),
                          ROW(trunc, n0, T), ROW(tv, n0, T), gamma, lam, ROW(adv, n0, T),
                          ROW(targets, n0, T), NULL, NULL, NULL) != 0;
    });
}

int oracle_rows_td_lambda(int nthreads, int64_t N, int64_t T, const double *r,
                          const double *v, const uint8_t *term, const uint8_t *trunc,
                          const double *tv, double gamma, double lam, double *ret)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_td_lambda(n, T, ROW(r, n0, T), ROW(v, n0, T + 1), ROW(term, n0, T),
                                ROW(trunc, n0, T), ROW(tv, n0, T), gamma, lam,
                                ROW(ret, n0, T), NULL, NULL, NULL) != 0;
    });
}

int oracle_rows_vtrace(int nthreads, int64_t N, int64_t T, const double *r, const double *v,
                       const double *log_rho, const uint8_t *term, const uint8_t *trunc,
                       const double *tv, double gamma, double lam, double rho_bar,
                       double c_bar, double pg_rho_bar, double *vs, double *pg)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_vtrace(n, T, ROW(r, n0, T), ROW(v, n0, T + 1), ROW(log_rho, n0, T),
                             ROW(term, n0, T), ROW(trunc, n0, T), ROW(tv, n0, T), gamma, lam,
                             rho_bar, c_bar, pg_rho_bar, ROW(vs, n0, T), ROW(pg, n0, T),
                             NULL, NULL, NULL) != 0;
    });
}

int oracle_rows_retrace(int nthreads, int64_t N, int64_t T, const double *r, const double *q,
                        const double *eq, const double *log_rho, const uint8_t *term,
                        const uint8_t *trunc, double gamma, double lam, double c_bar,
                        double *qret)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_retrace(n, T, ROW(r, n0, T), ROW(q, n0, T), ROW(eq, n0, T),
                              ROW(log_rho, n0, T), ROW(term, n0, T), ROW(trunc, n0, T), gamma,
                              lam, c_bar, ROW(qret, n0, T), NULL, NULL, NULL) != 0;
    });
}

int oracle_rows_eligibility_trace(int nthreads, int64_t N, int64_t T, const double *x,
                                  const uint8_t *term, const uint8_t *trunc,
                                  const double *z_init, double gamma, double lam, double *z)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_eligibility_trace(n, T, ROW(x, n0, T), ROW(term, n0, T),
                                        ROW(trunc, n0, T), ROW(z_init, n0, 1), gamma, lam,
                                        ROW(z, n0, T), NULL, NULL) != 0;
    });
}

int oracle_rows_episodic_cumsum(int nthreads, int64_t N, int64_t T, const double *x,
                                const uint8_t *term, const uint8_t *trunc,
                                const double *s_init, double *s)
{
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_episodic_cumsum(n, T, ROW(x, n0, T), ROW(term, n0, T), ROW(trunc, n0, T),
                                      ROW(s_init, n0, 1), ROW(s, n0, T), NULL, NULL) != 0;
    });
}

int oracle_rows_retrace_probs(int nthreads, int64_t N, int64_t T, int64_t A, const double *r,
                              const double *q, const int32_t *actions, const double *log_pi,
                              const double *log_mu, int mu_taken, const uint8_t *term,
                              const uint8_t *trunc, const double *trunc_eq, double gamma,
                              double lam, double c_bar, double *qret)
{
    const int64_t ld_tab = (T + 1) * A, ld_mu = mu_taken ? T : T * A;
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_retrace_probs(n, T, A, ROW(r, n0, T), ROW(q, n0, ld_tab),
                                    ROW(actions, n0, T), ROW(log_pi, n0, ld_tab),
                                    ROW(log_mu, n0, ld_mu), mu_taken, ROW(term, n0, T),
                                    ROW(trunc, n0, T), ROW(trunc_eq, n0, T), gamma, lam, c_bar,
                                    ROW(qret, n0, T), NULL, NULL, NULL) != 0;
    });
}

int oracle_rows_vtrace_probs(int nthreads, int64_t N, int64_t T, int64_t A, const double *r,
                             const double *v, const int32_t *actions, const double *log_pi,
                             const double *log_mu, int mu_taken, const uint8_t *term,
                             const uint8_t *trunc, const double *tv, double gamma, double lam,
                             double rho_bar, double c_bar, double pg_rho_bar, double *vs,
                             double *pg)
{
    const int64_t ld_mu = mu_taken ? T : T * A;
    FOR_SLICES(N, nthreads, {
        rc_ |= oracle_vtrace_probs(n, T, A, ROW(r, n0, T), ROW(v, n0, T + 1),
                                   ROW(actions, n0, T), ROW(log_pi, n0, T * A),
                                   ROW(log_mu, n0, ld_mu), mu_taken, ROW(term, n0, T),
                                   ROW(trunc, n0, T), ROW(tv, n0, T), gamma, lam, rho_bar,
                                   c_bar, pg_rho_bar, ROW(vs, n0, T), ROW(pg, n0, T), NULL, NULL,
                                   NULL) != 0;
    });
}
