/*
 * rlca.h -- reverse linear recurrences for RL credit assignment on AMD
 * Instinct MI355X (gfx950).  C ABI of librlca.so.
 *
 * Every entry point evaluates one first-order affine recurrence, in reverse
 * time
 *
 *     A_t = alpha_t + beta_t * A_{t+1},      t = T-1 ... 0,           (R)
 *
 * (the forward-time mirrors and the generic scan also run it forward,
 * A_t = alpha_t + beta_t * A_{t-1}), independently for each of num_envs rows,
 * as stated in the rl-triton
 * explainer pages ("rl-triton: High-Performance Triton GPU Kernels for
 * Reinforcement Learning Credit Assignment", Zehnder 2026; Technical summary,
 * Method 1, "Unified algebraic framework").  The GPU evaluates (R) as an
 * associative scan over the affine pairs (alpha_t, beta_t) with the operator
 *     (alpha_B, beta_B) (+) (alpha_A, beta_A) = (alpha_B + beta_B alpha_A, beta_A beta_B)
 * (same section), building the pairs and the outputs in registers in a single
 * pass over the inputs (Method 2, "Fused kernels").
 *
 * Episode boundaries (Method 3, "Explicit boundary semantics"), per row and
 * step t:
 *   term_t   terminated[t] != 0: natural end; the successor value is 0.
 *   trunc_t  truncated[t]  != 0: time limit; the successor value is the
 *            supplied bootstrap trunc_values[t] (the value of the true final
 *            observation).  A step flagged both ways counts as terminated.
 *   Either flag cuts the trace: beta_t = 0, so nothing after step t reaches
 *   any output at or before t.
 *   Rollout window end (t = T-1): the window bootstrap enters either
 *   alpha_{T-1} (GAE, TD(lambda), V-trace, Retrace) or the carry A_T
 *   (discounted returns), never both.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array pointer is a device pointer (memory the GPU of
 *   `stream` can read or write: hipMalloc'd or torch CUDA tensors).  `stream`
 *   is a hipStream_t passed as void*; NULL means the default stream.
 * Layout.  Row-major [num_envs, T] (values: [num_envs, T+1]); `ld_*` is the
 *   distance between rows in elements (>= T, or >= T+1 for values); elements
 *   along T are contiguous.  No alignment beyond the element size is
 *   required.  Flags are uint8 (torch.bool compatible), nonzero = true.
 *   Limits: num_envs <= 2^31-1, T <= 2^31-2, every ld <= 2^31-1.
 *   trunc_values must be a valid [num_envs, T] array when truncated is
 *   given, but only its entries at truncated (and not terminated) steps
 *   affect any output; the others may hold anything, NaN included.  Small
 *   batches read it in full, large ones only at truncated steps.
 * dtype.  RLCA_F32 or RLCA_BF16 gives the type of EVERY floating-point input
 *   array of the call (rewards, values, trunc_values, log_rhos, q_taken,
 *   exp_q_next, bootstrap, z_init, s_init, x, alpha, beta, q_values, log_pi,
 *   log_mu, trunc_eq), except the window calls' carry vectors, which are
 *   always fp32.  Arithmetic is fp32; outputs are always fp32.  Actions are
 *   int32.
 * Ownership.  The caller owns every buffer, the split calls' workspace
 *   included.  The library allocates no memory, keeps no state between calls
 *   (a per-thread tiling override, rlca_set_variant, aside), never
 *   synchronizes, and returns as soon as the work is enqueued on `stream`.
 * Nullable inputs.  terminated == NULL means no terminations; truncated ==
 *   NULL means no truncations (trunc_values is then ignored and may be NULL).
 * Non-finite inputs.  Episode boundaries cut the recurrence with a zero
 *   factor (A_t = alpha_t + 0 * A_{t+1}), and 0 * NaN = 0 * inf = NaN: a NaN
 *   or infinite input the recurrence reaches makes every output on its far
 *   side in scan order (earlier steps; later ones for the forward mirrors)
 *   of its row non-finite, across episode boundaries too.  Finite values
 *   never cross a boundary.
 * Errors.  Arguments are validated before anything is enqueued; on any
 *   non-OK status nothing is launched and no output is written (the one
 *   exception, a launch refused in the middle of a split call, is stated
 *   with the split calls below).
 *     T < 1                          -> RLCA_EINVAL (also when num_envs == 0).
 *     num_envs == 0                  -> RLCA_OK, nothing launched.
 *     negative num_envs, NULL required pointer, ld too small, misaligned pointer,
 *     gamma or lam outside [0, 1] or NaN, clip <= 0 or NaN,
 *     truncated != NULL with trunc_values == NULL  -> RLCA_EINVAL
 *     dtype other than RLCA_F32 / RLCA_BF16 -> RLCA_EDTYPE
 *     an output overlapping an input or another output -> RLCA_EALIAS
 *     the HIP runtime refusing the launch -> RLCA_EHIP
 *   rlca_last_error() returns a message for the calling thread's last
 *   non-OK status.  Device faults are asynchronous and surface at the
 *   caller's next synchronization with `stream`.
 * Concurrency.  Calls are thread-safe; calls on different streams may run
 *   concurrently if their outputs do not overlap.
 */
#ifndef RLCA_H
#define RLCA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RLCA_OK = 0,
    RLCA_EINVAL = 1,
    RLCA_EDTYPE = 2,
    RLCA_EALIAS = 3,
    RLCA_EHIP = 4
} rlca_status;

typedef enum {
    RLCA_F32 = 0,
    RLCA_BF16 = 1
} rlca_dtype;

/*
 * Discounted returns (Method 1, "discounted returns"):
 *   G_t = r_t + gamma * G_{t+1}           inside an episode,
 *   G_t = r_t                             if term_t,
 *   G_t = r_t + gamma * trunc_values[t]   if trunc_t (and not term_t),
 *   G_T = bootstrap[row]                  (the carry; bootstrap == NULL -> 0).
 * As (R): alpha_t = r_t + gamma*[trunc_t & !term_t]*trunc_values[t],
 *         beta_t = gamma*(1 - done_t).
 * In:  rewards [N,T]; bootstrap [N] (nullable, dtype of the call).
 * Out: returns [N,T] fp32.
 */
int rlca_returns(int64_t num_envs, int64_t T, int dtype,
                 const void *rewards, int64_t ld_rewards,
                 const uint8_t *terminated, int64_t ld_terminated,
                 const uint8_t *truncated, int64_t ld_truncated,
                 const void *trunc_values, int64_t ld_trunc_values,
                 const void *bootstrap,
                 float gamma,
                 float *returns, int64_t ld_returns,
                 void *stream);

/*
 * Generalized advantage estimation (Method 1, "GAE"; Schulman et al. 2016):
 *   next_t  = 0 if term_t; trunc_values[t] if trunc_t; values[t+1] otherwise
 *   delta_t = r_t + gamma * next_t - values[t]
 *   A_t     = delta_t + gamma*lam*(1 - done_t) * A_{t+1},   A_T = 0
 * values[T] (column T) is the window bootstrap and enters delta_{T-1} only.
 * In:  rewards [N,T], values [N,T+1], trunc_values [N,T] (used only where
 *      truncated and not terminated).
 * Out: advantages [N,T] fp32; targets [N,T] fp32 = A_t + values[t]
 *      (targets may be NULL).
 */
int rlca_gae(int64_t num_envs, int64_t T, int dtype,
             const void *rewards, int64_t ld_rewards,
             const void *values, int64_t ld_values,
             const uint8_t *terminated, int64_t ld_terminated,
             const uint8_t *truncated, int64_t ld_truncated,
             const void *trunc_values, int64_t ld_trunc_values,
             float gamma, float lam,
             float *advantages, int64_t ld_advantages,
             float *targets, int64_t ld_targets,
             void *stream);

/*
 * TD(lambda) returns (Method 1, "TD(lambda) returns"): the lambda-return
 *   G_t = A_t + values[t], with A_t the GAE advantage of rlca_gae on the same
 *   inputs.  Arguments as rlca_gae.
 * Out: lambda_returns [N,T] fp32.
 */
int rlca_td_lambda(int64_t num_envs, int64_t T, int dtype,
                   const void *rewards, int64_t ld_rewards,
                   const void *values, int64_t ld_values,
                   const uint8_t *terminated, int64_t ld_terminated,
                   const uint8_t *truncated, int64_t ld_truncated,
                   const void *trunc_values, int64_t ld_trunc_values,
                   float gamma, float lam,
                   float *lambda_returns, int64_t ld_lambda_returns,
                   void *stream);

/*
 * V-trace (Method 1, "V-trace"; Espeholt et al. 2018, eq. 1, with the
 * lambda-scaled trace):
 *   ratio_t = exp(log_rhos[t])  (log pi - log mu of the taken action)
 *   rho_t   = min(rho_bar, ratio_t),   c_t = lam * min(c_bar, ratio_t)
 *   A_t     = rho_t * delta_t + gamma * c_t * (1 - done_t) * A_{t+1},  A_T = 0
 *   vs_t    = values[t] + A_t
 *   pg_t    = min(pg_rho_bar, ratio_t) * (r_t + gamma * nvs_t - values[t]),
 *             nvs_t = 0 if term_t; trunc_values[t] if trunc_t;
 *                     vs_{t+1} otherwise (values[T] at t = T-1).
 * delta_t as in rlca_gae.  Clips must be > 0 (+inf allowed: no clipping).
 * In:  rewards [N,T], values [N,T+1], log_rhos [N,T], trunc_values [N,T].
 * Out: vs [N,T] fp32; pg_advantages [N,T] fp32 (nullable).
 */
int rlca_vtrace(int64_t num_envs, int64_t T, int dtype,
                const void *rewards, int64_t ld_rewards,
                const void *values, int64_t ld_values,
                const void *log_rhos, int64_t ld_log_rhos,
                const uint8_t *terminated, int64_t ld_terminated,
                const uint8_t *truncated, int64_t ld_truncated,
                const void *trunc_values, int64_t ld_trunc_values,
                float gamma, float lam, float rho_bar, float c_bar, float pg_rho_bar,
                float *vs, int64_t ld_vs,
                float *pg_advantages, int64_t ld_pg_advantages,
                void *stream);

/*
 * Retrace(lambda) (Method 1, "Retrace(lambda)"; Munos et al. 2016):
 *   c_t     = lam * min(c_bar, exp(log_rhos[t]))
 *   delta_t = r_t + gamma * (1 - term_t) * exp_q_next[t] - q_taken[t]
 *   A_t     = delta_t + gamma * c_{t+1} * (1 - done_t) * A_{t+1}  (t < T-1)
 *   A_{T-1} = delta_{T-1}   (c_T and Q_T lie outside the window)
 *   q_ret_t = q_taken[t] + A_t
 * q_taken[t] = Q(s_t, a_t); exp_q_next[t] = E_pi Q(s_{t+1}, .), which at a
 * truncation is the value of the true final state (kept; only the trace is
 * cut) and after a termination is ignored.  No trunc_values argument.
 * In:  rewards, q_taken, exp_q_next, log_rhos: [N,T].
 * Out: q_ret [N,T] fp32.
 */
int rlca_retrace(int64_t num_envs, int64_t T, int dtype,
                 const void *rewards, int64_t ld_rewards,
                 const void *q_taken, int64_t ld_q_taken,
                 const void *exp_q_next, int64_t ld_exp_q_next,
                 const void *log_rhos, int64_t ld_log_rhos,
                 const uint8_t *terminated, int64_t ld_terminated,
                 const uint8_t *truncated, int64_t ld_truncated,
                 float gamma, float lam, float c_bar,
                 float *q_ret, int64_t ld_q_ret,
                 void *stream);

/*
 * Forward-time mirrors of (R) (Method 1: "eligibility traces" and "episodic
 * prefix sums", computed forward in time):
 *     A_t = alpha_t + beta_t * A_{t-1},   t = 0 .. T-1,
 * with alpha_t = x_t.  A boundary after step t-1 (done_{t-1} = terminated or
 * truncated at t-1; the two are not distinguished here) restarts the
 * recurrence at step t: beta_t = 0.  A_{-1} is the per-row carry-in
 * (`z_init` / `s_init`, [N] in the call's dtype, NULL: 0), used as given
 * (zero it if the previous window ended an episode).
 *
 * Accumulating eligibility trace: beta_t = gamma * lam * (1 - done_{t-1}),
 *   z_t = x_t + gamma*lam*(1 - done_{t-1}) * z_{t-1}.
 * In:  x [N,T].  Out: traces [N,T] fp32.
 */
int rlca_eligibility_trace(int64_t num_envs, int64_t T, int dtype,
                           const void *x, int64_t ld_x,
                           const uint8_t *terminated, int64_t ld_terminated,
                           const uint8_t *truncated, int64_t ld_truncated,
                           const void *z_init,
                           float gamma, float lam,
                           float *traces, int64_t ld_traces,
                           void *stream);

/*
 * Episodic prefix sum: beta_t = 1 - done_{t-1},
 *   S_t = x_t + (1 - done_{t-1}) * S_{t-1}   (the running sum of x within
 *   each episode, e.g. the return so far).
 * In:  x [N,T].  Out: sums [N,T] fp32.
 */
int rlca_episodic_cumsum(int64_t num_envs, int64_t T, int dtype,
                         const void *x, int64_t ld_x,
                         const uint8_t *terminated, int64_t ld_terminated,
                         const uint8_t *truncated, int64_t ld_truncated,
                         const void *s_init,
                         float *sums, int64_t ld_sums,
                         void *stream);

/*
 * The materialized doubling scan (Problem: the vectorized O(log T) scan that
 * writes its intermediates to HBM and reads them back at every step, the
 * baseline the pages measure the fused kernels against; Method 2, Results).
 * Re-created in HIP so that the comparison can be made on MI355X; a
 * reference point, not a faster path.  rlca_X_materialized computes what
 * rlca_X computes (same arguments, same results up to rounding order, same
 * validation), in 2 + ceil(log2 T) kernel launches instead of one:
 *   1. (alpha_t, beta_t) of every step, as the coefficient table of rlca_X
 *      states them, written to the workspace;
 *   2. for s = 1, 2, 4, ... < T: every step composes its pair with the pair
 *      s steps later, (a_t, b_t) <- (a_t + b_t a_{t+s}, b_t b_{t+s}) where
 *      t + s < T, from one pair of arrays into the other;
 *   3. A_t = a_t + b_t A_T (A_T: returns' bootstrap, else 0) and the outputs.
 * Each launch streams whole [N, T] arrays through HBM: at T = 128, about 9
 * times the bytes of the fused call.
 * Workspace.  Device memory owned by the caller, 4-byte aligned, at least
 * rlca_materialized_workspace_bytes(N, T) = 16 N T bytes (two pairs of fp32
 * [N, T] arrays), not overlapping the call's arrays (RLCA_EALIAS); NULL or
 * smaller -> RLCA_EINVAL.  Calls sharing a workspace must be ordered.
 * rlca_materialized_workspace_bytes: -1 for num_envs < 0, T < 1, or a size
 * past 2^63 bytes.
 */
int64_t rlca_materialized_workspace_bytes(int64_t num_envs, int64_t T);
int rlca_returns_materialized(int64_t num_envs, int64_t T, int dtype,
                              const void *rewards, int64_t ld_rewards,
                              const uint8_t *terminated, int64_t ld_terminated,
                              const uint8_t *truncated, int64_t ld_truncated,
                              const void *trunc_values, int64_t ld_trunc_values,
                              const void *bootstrap,
                              float gamma,
                              float *returns, int64_t ld_returns,
                              void *workspace, int64_t workspace_bytes,
                              void *stream);
int rlca_gae_materialized(int64_t num_envs, int64_t T, int dtype,
                          const void *rewards, int64_t ld_rewards,
                          const void *values, int64_t ld_values,
                          const uint8_t *terminated, int64_t ld_terminated,
                          const uint8_t *truncated, int64_t ld_truncated,
                          const void *trunc_values, int64_t ld_trunc_values,
                          float gamma, float lam,
                          float *advantages, int64_t ld_advantages,
                          float *targets, int64_t ld_targets,
                          void *workspace, int64_t workspace_bytes,
                          void *stream);
int rlca_td_lambda_materialized(int64_t num_envs, int64_t T, int dtype,
                                const void *rewards, int64_t ld_rewards,
                                const void *values, int64_t ld_values,
                                const uint8_t *terminated, int64_t ld_terminated,
                                const uint8_t *truncated, int64_t ld_truncated,
                                const void *trunc_values, int64_t ld_trunc_values,
                                float gamma, float lam,
                                float *lambda_returns, int64_t ld_lambda_returns,
                                void *workspace, int64_t workspace_bytes,
                                void *stream);
int rlca_vtrace_materialized(int64_t num_envs, int64_t T, int dtype,
                             const void *rewards, int64_t ld_rewards,
                             const void *values, int64_t ld_values,
                             const void *log_rhos, int64_t ld_log_rhos,
                             const uint8_t *terminated, int64_t ld_terminated,
                             const uint8_t *truncated, int64_t ld_truncated,
                             const void *trunc_values, int64_t ld_trunc_values,
                             float gamma, float lam, float rho_bar, float c_bar,
                             float pg_rho_bar,
                             float *vs, int64_t ld_vs,
                             float *pg_advantages, int64_t ld_pg_advantages,
                             void *workspace, int64_t workspace_bytes,
                             void *stream);
int rlca_retrace_materialized(int64_t num_envs, int64_t T, int dtype,
                              const void *rewards, int64_t ld_rewards,
                              const void *q_taken, int64_t ld_q_taken,
                              const void *exp_q_next, int64_t ld_exp_q_next,
                              const void *log_rhos, int64_t ld_log_rhos,
                              const uint8_t *terminated, int64_t ld_terminated,
                              const uint8_t *truncated, int64_t ld_truncated,
                              float gamma, float lam, float c_bar,
                              float *q_ret, int64_t ld_q_ret,
                              void *workspace, int64_t workspace_bytes,
                              void *stream);

/*
 * Window entry points (Method 3, "rollout windows"; Method 1: the operator is
 * associative, so a rollout can be cut along time and the pieces chained).
 * A rollout longer than one call -- streamed as it is collected, or cut into
 * pieces evaluated apart -- is processed as consecutive windows of one
 * rollout.  Each rlca_X_chunk call takes the arguments of rlca_X (the
 * per-row bootstrap / initial value of returns and of the forward mirrors is
 * replaced by carry_in) plus three per-row fp32 vectors, whatever `dtype`,
 * and an optional workspace (workspace, workspace_bytes; NULL, 0: none) that
 * lets a call on few long rows run split (see "Split calls" below):
 *
 *   carry_in  [num_envs], nullable (0): the scan state A entering the window
 *             from the neighbouring window -- the later one for reverse
 *             recurrences (A_T), the earlier one for forward ones (A_{-1}).
 *   carry_out [num_envs], nullable: the value to pass as carry_in to the
 *             window on the other side (earlier for reverse, later for
 *             forward).  Like every output it must not overlap an input,
 *             carry_in included (RLCA_EALIAS): stream through two carry
 *             vectors used in turn.
 *   carry_map [num_envs, 2] (row-major pairs (a, b)), nullable: the affine
 *             map carry_out = a + b * carry_in of the window, whatever
 *             carry_in is.  With it, windows can be evaluated in parallel
 *             from carry 0 and joined afterwards: compose the maps from the
 *             far end to get each window's true carry_in, then evaluate the
 *             windows again with it.
 *
 * What the carry is, per algorithm (A as in each entry point above):
 *   returns       A = G.  carry_in = G_T (the bootstrap); carry_out = G_0.
 *   gae           A = advantage.  carry_in = A_T, the advantage of the step
 *                 after the window; carry_out = A_0.  values keeps its T+1
 *                 columns: V_T is the first value of the next window.
 *   td_lambda     A = G^lambda - V.  carry_in = G^lambda_T - V_T;
 *                 carry_out = G^lambda_0 - V_0 (= lambda_returns[0] - V_0).
 *   vtrace        A = vs - V.  carry_in = vs_T - V_T, which also enters pg at
 *                 step T-1 through vs_T; carry_out = vs_0 - V_0.
 *   retrace       A = q_ret - q_taken; the trace factor c_{t+1} multiplies
 *                 A_{t+1}, so the carry holds it: carry_in =
 *                 c_T (q_ret_T - q_taken_T) with c_T = lam min(c_bar,
 *                 exp(log_rho_T)) of the next window's first step, and
 *                 carry_out = c_0 (q_ret_0 - q_taken_0).  With carry_in NULL
 *                 the result equals rlca_retrace's.
 *   eligibility_trace, episodic_cumsum
 *                 carry_in = A_{-1} (z_init / s_init as fp32); carry_out =
 *                 A_{T-1}, or 0 if an episode ends after step T-1.
 * Splitting a rollout at any step and chaining the windows this way
 * reproduces the one-window result up to fp32 rounding.  Errors and
 * everything else as for rlca_X.  A window call with carry_in, carry_out and
 * carry_map all NULL computes what rlca_X computes (returns and the forward
 * mirrors: with a zero bootstrap / initial value).
 */
int rlca_returns_chunk(int64_t num_envs, int64_t T, int dtype,
                       const void *rewards, int64_t ld_rewards,
                       const uint8_t *terminated, int64_t ld_terminated,
                       const uint8_t *truncated, int64_t ld_truncated,
                       const void *trunc_values, int64_t ld_trunc_values,
                       const float *carry_in, float gamma,
                       float *returns, int64_t ld_returns,
                       float *carry_out, float *carry_map,
                       void *workspace, int64_t workspace_bytes,
                       void *stream);
int rlca_gae_chunk(int64_t num_envs, int64_t T, int dtype,
                   const void *rewards, int64_t ld_rewards,
                   const void *values, int64_t ld_values,
                   const uint8_t *terminated, int64_t ld_terminated,
                   const uint8_t *truncated, int64_t ld_truncated,
                   const void *trunc_values, int64_t ld_trunc_values,
                   float gamma, float lam,
                   float *advantages, int64_t ld_advantages,
                   float *targets, int64_t ld_targets,
                   const float *carry_in, float *carry_out, float *carry_map,
                   void *workspace, int64_t workspace_bytes,
                   void *stream);
/*
 * rlca_gae_chunk_noalloc: rlca_gae_chunk for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments without
 * (workspace, workspace_bytes), same results: a call that would split (see
 * "Split calls" below) takes the three-launch form, with its workspace from
 * a 6 KB array that the library holds on each device until the process
 * ends, room for every split of that form (3 floats per segment, at most 512
 * segments; a larger need is RLCA_EINVAL).  The array's address on a device is looked up on the
 * first call there (with that device made current for the lookup); no call
 * allocates or frees memory.  Every call on one device shares that device's
 * array, and each split call overwrites it before reading it: calls that
 * overlap in time on one device (different streams) race and must not be
 * made; calls on one stream are ordered.  An unsplit call does not touch it.
 */
int rlca_gae_chunk_noalloc(int64_t num_envs, int64_t T, int dtype,
                           const void *rewards, int64_t ld_rewards,
                           const void *values, int64_t ld_values,
                           const uint8_t *terminated, int64_t ld_terminated,
                           const uint8_t *truncated, int64_t ld_truncated,
                           const void *trunc_values, int64_t ld_trunc_values,
                           float gamma, float lam,
                           float *advantages, int64_t ld_advantages,
                           float *targets, int64_t ld_targets,
                           const float *carry_in, float *carry_out, float *carry_map,
                           void *stream);
int rlca_td_lambda_chunk(int64_t num_envs, int64_t T, int dtype,
                         const void *rewards, int64_t ld_rewards,
                         const void *values, int64_t ld_values,
                         const uint8_t *terminated, int64_t ld_terminated,
                         const uint8_t *truncated, int64_t ld_truncated,
                         const void *trunc_values, int64_t ld_trunc_values,
                         float gamma, float lam,
                         float *lambda_returns, int64_t ld_lambda_returns,
                         const float *carry_in, float *carry_out, float *carry_map,
                         void *workspace, int64_t workspace_bytes,
                         void *stream);
int rlca_vtrace_chunk(int64_t num_envs, int64_t T, int dtype,
                      const void *rewards, int64_t ld_rewards,
                      const void *values, int64_t ld_values,
                      const void *log_rhos, int64_t ld_log_rhos,
                      const uint8_t *terminated, int64_t ld_terminated,
                      const uint8_t *truncated, int64_t ld_truncated,
                      const void *trunc_values, int64_t ld_trunc_values,
                      float gamma, float lam, float rho_bar, float c_bar, float pg_rho_bar,
                      float *vs, int64_t ld_vs,
                      float *pg_advantages, int64_t ld_pg_advantages,
                      const float *carry_in, float *carry_out, float *carry_map,
                      void *workspace, int64_t workspace_bytes,
                      void *stream);
int rlca_retrace_chunk(int64_t num_envs, int64_t T, int dtype,
                       const void *rewards, int64_t ld_rewards,
                       const void *q_taken, int64_t ld_q_taken,
                       const void *exp_q_next, int64_t ld_exp_q_next,
                       const void *log_rhos, int64_t ld_log_rhos,
                       const uint8_t *terminated, int64_t ld_terminated,
                       const uint8_t *truncated, int64_t ld_truncated,
                       float gamma, float lam, float c_bar,
                       float *q_ret, int64_t ld_q_ret,
                       const float *carry_in, float *carry_out, float *carry_map,
                       void *workspace, int64_t workspace_bytes,
                       void *stream);
int rlca_eligibility_trace_chunk(int64_t num_envs, int64_t T, int dtype,
                                 const void *x, int64_t ld_x,
                                 const uint8_t *terminated, int64_t ld_terminated,
                                 const uint8_t *truncated, int64_t ld_truncated,
                                 const float *carry_in,
                                 float gamma, float lam,
                                 float *traces, int64_t ld_traces,
                                 float *carry_out, float *carry_map,
                                 void *workspace, int64_t workspace_bytes,
                                 void *stream);
int rlca_episodic_cumsum_chunk(int64_t num_envs, int64_t T, int dtype,
                               const void *x, int64_t ld_x,
                               const uint8_t *terminated, int64_t ld_terminated,
                               const uint8_t *truncated, int64_t ld_truncated,
                               const float *carry_in,
                               float *sums, int64_t ld_sums,
                               float *carry_out, float *carry_map,
                               void *workspace, int64_t workspace_bytes,
                               void *stream);

/*
 * Generic segmented affine scan: (R) itself with caller-given coefficients
 * (Method 1: every entry point above is an instance of it; the pages'
 * "Significance and claims" section names long-context LLM post-training and
 * spiking neural networks as further uses of the same fused scan).
 *   reverse = 1:  A_t = alpha_t + beta'_t * A_{t+1},  t = T-1 .. 0,  A_T = carry_in
 *   reverse = 0:  A_t = alpha_t + beta'_t * A_{t-1},  t = 0 .. T-1,  A_{-1} = carry_in
 * beta'_t = 0 where reset[t] != 0 (step t starts a segment: nothing flows in
 * from its neighbour), beta_t elsewhere; reset NULL: no resets.
 * In:  alpha, beta [N,T] (dtype), reset [N,T] uint8 (nullable).
 * Out: out [N,T] fp32 (= A).  carry_in, carry_out, carry_map and the
 * workspace as for the window entry points: carry_out is A_0 (reverse) or
 * A_{T-1} (forward), as is; a reset at the next window's first step belongs
 * to that window.
 * reverse other than 0 or 1 -> RLCA_EINVAL.
 */
int rlca_affine_scan(int64_t num_envs, int64_t T, int dtype,
                     const void *alpha, int64_t ld_alpha,
                     const void *beta, int64_t ld_beta,
                     const uint8_t *reset, int64_t ld_reset,
                     int reverse,
                     const float *carry_in,
                     float *out, int64_t ld_out,
                     float *carry_out, float *carry_map,
                     void *workspace, int64_t workspace_bytes,
                     void *stream);

/*
 * Retrace(lambda) and V-trace from the policies' log-probability tables
 * (Results: the heavier Retrace workload loads the action probabilities at
 * every step).  With A = num_actions and a_t = actions[t] (int32, the action
 * taken at step t):
 *   log_rho_t = log_pi[t][a_t] - log_mu[t][a_t]
 * replaces the log_rhos input of rlca_retrace / rlca_vtrace, and Retrace
 * forms its other per-step inputs on chip:
 *   q_taken_t  = q_values[t][a_t]
 *   exp_q_next_t = sum over a of exp(log_pi[t+1][a]) * q_values[t+1][a]
 *                  (E_pi Q(s_{t+1}, .)), except after a truncation that is not
 *                  a termination, where the tables' slice t+1 is the next
 *                  episode's first state: trunc_eq[t] (E_pi Q at the true final
 *                  state, supplied; read only there).
 * Everything else is as for rlca_retrace / rlca_vtrace (same outputs, same
 * boundary rules, same tolerances).  Determinism: V-trace is bit-reproducible
 * run to run; Retrace's expectation is summed in an order that can vary
 * between runs (on-chip atomic adds), so its outputs can differ in the last
 * bits between otherwise identical calls.
 * Layout.  A table is row-major [num_envs, S, A] with S slices per row, A
 *   entries per slice contiguous; ld_* is the distance between rows in
 *   elements (>= S * A).  Retrace: q_values and log_pi have S = T + 1 (slice
 *   T is the state after the window), log_mu S = T.  V-trace: log_pi and
 *   log_mu have S = T.  actions is [num_envs, T] int32.  log_mu_taken = 1:
 *   log_mu is instead [num_envs, T] (row stride ld_log_mu >= T) holding
 *   log mu(a_t | s_t) of the taken actions only, the form replay buffers
 *   usually keep; the full table costs a whole read of it.  0 or 1, else
 *   RLCA_EINVAL.
 * Errors.  As for the other entry points; also num_actions outside
 *   [1, 65536] -> RLCA_EINVAL, and (Retrace) truncated != NULL with
 *   trunc_eq == NULL -> RLCA_EINVAL.  An action outside [0, A) is not
 *   detected before launch and reads no memory outside the tables: its step
 *   and every earlier step of its row come out NaN (the scan cuts episodes
 *   by a zero factor, which does not stop a NaN), later steps are unaffected.
 * Rows of more than 256 steps are processed by one 256-thread workgroup
 * each, 1024 steps per tile; shorter rows by one wavefront each, four rows
 * per workgroup.  The tiling controls do not apply (rlca_last_variant()
 * reports -1).
 */
int rlca_retrace_probs(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                       const void *rewards, int64_t ld_rewards,
                       const void *q_values, int64_t ld_q_values,
                       const int32_t *actions, int64_t ld_actions,
                       const void *log_pi, int64_t ld_log_pi,
                       const void *log_mu, int64_t ld_log_mu, int log_mu_taken,
                       const uint8_t *terminated, int64_t ld_terminated,
                       const uint8_t *truncated, int64_t ld_truncated,
                       const void *trunc_eq, int64_t ld_trunc_eq,
                       float gamma, float lam, float c_bar,
                       float *q_ret, int64_t ld_q_ret,
                       void *stream);
int rlca_vtrace_probs(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                      const void *rewards, int64_t ld_rewards,
                      const void *values, int64_t ld_values,
                      const int32_t *actions, int64_t ld_actions,
                      const void *log_pi, int64_t ld_log_pi,
                      const void *log_mu, int64_t ld_log_mu, int log_mu_taken,
                      const uint8_t *terminated, int64_t ld_terminated,
                      const uint8_t *truncated, int64_t ld_truncated,
                      const void *trunc_values, int64_t ld_trunc_values,
                      float gamma, float lam, float rho_bar, float c_bar, float pg_rho_bar,
                      float *vs, int64_t ld_vs,
                      float *pg_advantages, int64_t ld_pg_advantages,
                      void *stream);

/*
 * Window forms of the two policy-table calls: the arguments of
 * rlca_retrace_probs / rlca_vtrace_probs followed by carry_in, carry_out and
 * carry_map, with the meanings of the window entry points above (Retrace:
 * c_T (q_ret_T - q_taken_T); V-trace: vs_T - V_T).
 */
int rlca_retrace_probs_chunk(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                             const void *rewards, int64_t ld_rewards,
                             const void *q_values, int64_t ld_q_values,
                             const int32_t *actions, int64_t ld_actions,
                             const void *log_pi, int64_t ld_log_pi,
                             const void *log_mu, int64_t ld_log_mu, int log_mu_taken,
                             const uint8_t *terminated, int64_t ld_terminated,
                             const uint8_t *truncated, int64_t ld_truncated,
                             const void *trunc_eq, int64_t ld_trunc_eq,
                             float gamma, float lam, float c_bar,
                             float *q_ret, int64_t ld_q_ret,
                             const float *carry_in, float *carry_out, float *carry_map,
                             void *stream);
int rlca_vtrace_probs_chunk(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                            const void *rewards, int64_t ld_rewards,
                            const void *values, int64_t ld_values,
                            const int32_t *actions, int64_t ld_actions,
                            const void *log_pi, int64_t ld_log_pi,
                            const void *log_mu, int64_t ld_log_mu, int log_mu_taken,
                            const uint8_t *terminated, int64_t ld_terminated,
                            const uint8_t *truncated, int64_t ld_truncated,
                            const void *trunc_values, int64_t ld_trunc_values,
                            float gamma, float lam, float rho_bar, float c_bar, float pg_rho_bar,
                            float *vs, int64_t ld_vs,
                            float *pg_advantages, int64_t ld_pg_advantages,
                            const float *carry_in, float *carry_out, float *carry_map,
                            void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *rlca_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int rlca_version(void);

/*
 * Tiling variants.  Each lane owns K consecutive steps.  K = 4 (one 16-byte
 * vector of every fp32 array and of every output) except in the wide
 * variants on bf16 inputs, where K = 8 (one 16-byte vector of every bf16
 * array) for every algorithm but V-trace; on fp32 inputs and for V-trace a
 * wide variant runs the same kernel as its narrow twin.  A variant fixes how
 * many lanes share one row within a wavefront, how many wavefronts cooperate
 * on one row, and whether it is wide; rows longer than a tile are processed
 * tile by tile.  Variants 0-2: 16, 32 or 64 lanes of one wavefront per row;
 * 3-5: 4, 8 or 16 wavefronts per row; 6-8: 3-5, wide.
 * By default each call picks one from (num_envs, T, dtype, algorithm).
 * rlca_set_variant(v) forces variant v (0 <= v < rlca_num_variants()) for
 * later calls on the calling thread, or restores the automatic choice with
 * v = -1; it returns the previous setting, or -2 for an unknown v (setting
 * unchanged).  Every variant computes the same results up to rounding order.
 * rlca_variant_info writes the steps per lane K of variant v for the
 * algorithm `algo` (an rlca_algo; a window form takes its algorithm's, the
 * affine scan RLCA_ALGO_AFFINE in either direction) and `dtype`, the number
 * of lanes that share one row (tile = K x lanes per row) and the wavefronts
 * per row, and returns RLCA_OK, or RLCA_EINVAL (unknown variant or
 * algorithm) / RLCA_EDTYPE.  rlca_last_variant() is the variant the calling
 * thread's last successful launch used (-1 if none).  The policy-table entry
 * points have their own tiling and are not described by these calls.
 */
typedef enum {
  RLCA_ALGO_RETURNS = 0,
  RLCA_ALGO_GAE = 1,
  RLCA_ALGO_TD_LAMBDA = 2,
  RLCA_ALGO_VTRACE = 3,
  RLCA_ALGO_RETRACE = 4,
  RLCA_ALGO_ELIGIBILITY = 5,
  RLCA_ALGO_CUMSUM = 6,
  RLCA_ALGO_AFFINE = 7
} rlca_algo;

/*
 * Split calls: few long rows (Method 1: the operator is associative, so a
 * row can be cut along time, its pieces scanned apart and joined by their
 * carry maps).  With one workgroup per row, a call on fewer rows than the
 * GPU's 256 compute units leaves some of them idle, and long rows keep the
 * others busy for long.  A window call of the scan family (rlca_*_chunk of
 * the seven algorithms and rlca_affine_scan; not the policy-table calls)
 * given a workspace then cuts every row into segments, in one of two forms,
 * and computes the same results up to rounding order:
 *
 * Chained (one pass), for N rows of T >= 8192 steps with N <= 224 and
 * N <= T / 128 (16384 steps: up to 128 rows; 32768 and more: 224).  The
 * segment length L is one or two whole tiles of a tiling with whole
 * wavefronts per row (rlca_variant_info: K x lanes per row steps per tile)
 * with T % L == 0 and 2 <= T / L <= 256; of those, with S = T / L, the one
 * with the least ceil(N * S / 256) * L + ceil(N * S / (256 * r)) * 4096
 * + 32 * S, ties going to the longer, where r is 1 for the 16-wavefront
 * two-tile segments of returns, GAE and TD(lambda) at K = 8, of V-trace,
 * and of Retrace at K = 8 or on bf16 inputs (a compute unit holds one such
 * workgroup at once), else 2.  On bf16 inputs (but for V-trace) the wide
 * tilings (K = 8) are taken where any of them gives such an L, the others
 * only otherwise.  Where such an L exists, the rows share one row stride,
 * and the workspace is 8-byte aligned and holds 8 bytes plus 32 per
 * segment: one launch, one workgroup per segment that reads the
 * workspace's epoch word (the previous call's tag; this call's is the next
 * value, never 0), scans its segment,
 * publishes its carry map in the workspace, composes the maps the segments
 * before it in scan order have published into the carry entering its own
 * (from the row's end for reverse recurrences, from its start for the
 * forward mirrors, starting at carry_in), publishes the map to the carry it
 * hands on, and writes its outputs; the launch's last workgroup then stores
 * the call's tag in the epoch word, once every workgroup has read it.  The
 * inputs are read once.  Published words carry the tag, so the workspace
 * needs no clearing, before the first call or between calls (also between
 * replays of a captured graph).  A workgroup waits only for workgroups
 * launched before it; its wait is bounded all the same, and a carry not
 * found within the bound (which the hardware's in-order workgroup dispatch
 * rules out) turns that segment's outputs into NaN.
 *
 * Three launches, otherwise, on at most 64 rows of at least 32768 steps:
 * S = rlca_split_segments(N, T) segments of T / S steps; the segments from carry 0, writing only their carry maps to
 * the workspace; a small kernel composing, per row, the carry that enters
 * each segment from carry_in, and the row's carry_out and carry_map; and the
 * segments again from those carries, writing the outputs.  It reads the
 * inputs twice.
 *
 * rlca_set_chained(0) makes the calling thread's split calls take the
 * three-launch form (for tests and comparisons); rlca_set_chained(1) restores
 * the default.  It returns the previous setting.  rlca_last_launches() is
 * the number of kernel launches the calling thread's last successful call
 * enqueued, rlca_last_segments() the number of segments it cut each row
 * into (1: not split; a chained call is one launch of more than one
 * segment).  The plain entry points (rlca_gae, ...) never split: for the
 * same result on few long rows call the window form with NULL carries and a
 * workspace.
 *
 * Workspace.  Device memory owned by the caller, 4-byte aligned (8 for the
 * chained form), at least rlca_split_workspace_bytes(N, T) bytes; it must not
 * overlap the call's arrays (RLCA_EALIAS).  It is used only when the call
 * splits (otherwise the call runs unsplit and never touches it); then a size
 * below what the three-launch form needs is RLCA_EINVAL (a size that fits
 * only that form selects it).  Calls that share a workspace must be ordered,
 * for instance issued to one stream: the library does not synchronize.
 * workspace_bytes < 0 or a misaligned workspace -> RLCA_EINVAL.
 *
 * Failure.  Every argument is validated before the first launch.  Kernel
 * launches cannot be withdrawn once enqueued, so should the runtime refuse
 * the second or third launch of the three-launch form (RLCA_EHIP, which a
 * launch that the runtime accepted on the same stream an instant earlier
 * leaves only to a failing runtime or device), the earlier launches stay
 * enqueued: the workspace and, after the second, carry_out and carry_map may
 * then hold results, while the outputs are not written.
 *
 * rlca_split_segments(num_envs, T) returns the three-launch form's S (1: no
 * split): the smallest power of two with num_envs * S >= 256, T divisible by
 * S and T / S >= 4096, stopping where either condition would fail; 1 for
 * more than 64 rows and for rows shorter than 32768 steps; -1 (with a message
 * for rlca_last_error) for num_envs < 0 or T < 1.
 * rlca_split_workspace_bytes(num_envs, T) returns the workspace a split call
 * may use, the larger of the three-launch form's 12 * num_envs * S bytes (3
 * floats per segment) and the chained form's 8 bytes plus 32 per segment for
 * any input dtype and algorithm, or 0 when neither splits; -1 as above.
 */
int rlca_split_segments(int64_t num_envs, int64_t T);
int64_t rlca_split_workspace_bytes(int64_t num_envs, int64_t T);

/*
 * Kernel timing (instrumented build only; a measurement tool, not part of
 * the computation).  librlca.so is built without it.  librlca_timed.so, built
 * from the same sources with RLCA_TIMESTAMPS defined (python -m
 * reverse_linear_recurrence_amd.build --timestamps), has every wavefront of
 * a scan kernel record the GPU's 100 MHz wall clock at entry and again once
 * all of its loads and stores have completed.  rlca_timestamps copies the
 * (start, end) pairs of the calling thread's last launch, one pair per
 * wavefront in launch order, for at most max_waves wavefronts (and at most
 * 65536), into dst (host memory, 2 * max_waves uint64), and sets *waves to
 * the number copied; the launch's duration on the GPU is then max(end) -
 * min(start) ticks of 10 ns.  It synchronizes with the device.  Only the
 * last launch of each device is kept: read it before launching again.
 * librlca.so: RLCA_EINVAL.
 */
int rlca_timestamps(uint64_t *dst, int64_t max_waves, int64_t *waves);

int rlca_num_variants(void);
int rlca_set_variant(int variant);
int rlca_variant_info(int variant, int algo, int dtype, int *steps_per_lane, int *lanes_per_row,
                      int *waves_per_row);
int rlca_last_variant(void);
int rlca_set_chained(int enable);
int rlca_last_launches(void);
int rlca_last_segments(void);

#ifdef __cplusplus
}
#endif

#endif /* RLCA_H */
