// rlca.hip -- host side of librlca.so: argument validation, tiling choice and
// kernel launch for the C ABI declared in include/rlca.h.
//
// Nothing here touches element data: every step of the computation runs in
// the kernels of scan_kernels.hpp.  A call validates its arguments, picks a
// tiling variant, and enqueues exactly one kernel on the caller's stream.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "rlca.h"
#include "scan_kernels.hpp"

namespace rlca {
namespace {

// ------------------------------------------------------------- variants

struct Variant {
  int LPR;  // lanes per row inside a wavefront (64 when WPR > 1)
  int WPR;  // wavefronts per row
};

// Every lane owns K = 4 consecutive steps: one 16-byte vector of each fp32
// array (an 8-byte vector of each bf16 array) and one 16-byte vector of each
// fp32 output, so every load and store instruction of a wavefront covers one
// contiguous span and uses each cache line it touches in full.  (Longer spans
// per lane split each instruction into strided partial lines: 4x the line
// requests for 16 fp32 steps per lane, and partial-line output writes for 8
// bf16 steps per lane.)
constexpr int kStepsPerLane = 4;
constexpr Variant kVariants[] = {
    {16, 1},  // 0: tile    64 steps, 16 rows per 256-thread workgroup
    {32, 1},  // 1: tile   128,  8 rows per workgroup
    {64, 1},  // 2: tile   256,  4 rows per workgroup
    {64, 4},  // 3: tile  1024,  1 row per 256-thread workgroup
    {64, 8},  // 4: tile  2048,  1 row per 512-thread workgroup
    {64, 16}, // 5: tile  4096,  1 row per 1024-thread workgroup
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int64_t tile_steps(const Variant &v, int /*dtype*/) {
  return static_cast<int64_t>(kStepsPerLane) * v.LPR * v.WPR;
}

template <int A, typename InT, int V, bool U>
const void *kernel_for() {
  constexpr Variant v = kVariants[V];
  return reinterpret_cast<const void *>(&scan_kernel<A, InT, kStepsPerLane, v.LPR, v.WPR, U>);
}

template <int A, typename InT, bool U>
const void *kernel_for(int v) {
  switch (v) {
    case 0: return kernel_for<A, InT, 0, U>();
    case 1: return kernel_for<A, InT, 1, U>();
    case 2: return kernel_for<A, InT, 2, U>();
    case 3: return kernel_for<A, InT, 3, U>();
    case 4: return kernel_for<A, InT, 4, U>();
    default: return kernel_for<A, InT, 5, U>();
  }
}

template <int A>
const void *kernel_for(int dtype, int v, bool uniform) {
  if (dtype == RLCA_BF16)
    return uniform ? kernel_for<A, bf16_t, true>(v) : kernel_for<A, bf16_t, false>(v);
  return uniform ? kernel_for<A, float, true>(v) : kernel_for<A, float, false>(v);
}

const void *kernel_for(int algo, int dtype, int v, bool uniform) {
  switch (algo) {
    case kReturns: return kernel_for<kReturns>(dtype, v, uniform);
    case kGae: return kernel_for<kGae>(dtype, v, uniform);
    case kTdLambda: return kernel_for<kTdLambda>(dtype, v, uniform);
    case kVtrace: return kernel_for<kVtrace>(dtype, v, uniform);
    case kRetrace: return kernel_for<kRetrace>(dtype, v, uniform);
    case kEligibility: return kernel_for<kEligibility>(dtype, v, uniform);
    default: return kernel_for<kCumsum>(dtype, v, uniform);
  }
}

// Default tiling (measured on MI355X).  Short rows: the smallest
// one-wavefront tile that covers T.  Long rows (tiles loop along T, each
// tile's loads issued while the previous one is computed): about 4096
// wavefronts (16 per CU) -- the most wavefronts per row such that N * WPR
// stays within that and the tile is not longer than the row; from 8192 rows
// on, one wavefront per row.
int auto_variant(int64_t N, int64_t T, int dtype) {
  constexpr int64_t kTargetWaves = 4096;
  for (int v = 0; v <= 2; ++v)
    if (T <= tile_steps(kVariants[v], dtype)) return v;
  if (N >= 2 * kTargetWaves) return 2;
  for (int v = kNumVariants - 1; v >= 3; --v)
    if (N * kVariants[v].WPR <= kTargetWaves && tile_steps(kVariants[v], dtype) <= T) return v;
  return tile_steps(kVariants[3], dtype) <= T ? 3 : 2;
}

// ------------------------------------------------------------- errors

thread_local std::string t_last_error;
thread_local int t_forced_variant = -1;
thread_local int t_last_variant = -1;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return status;
}

// ------------------------------------------------------------- validation

struct Arr {
  const char *name;
  const void *ptr;
  int64_t ld;      // row stride in elements
  int64_t width;   // elements used per row
  int64_t esize;   // bytes per element
  bool required;
  bool output;
  bool one_row = false;  // a single row (the per-row bootstrap vector)
  // Byte span [lo, hi) the call may touch; filled by check_array.
  uintptr_t lo = 0, hi = 0;
};

int check_array(Arr &a, int64_t N) {
  if (a.one_row) N = 1;
  if (a.ptr == nullptr) {
    if (a.required) return fail(RLCA_EINVAL, "%s must not be NULL", a.name);
    return RLCA_OK;
  }
  const uintptr_t p = reinterpret_cast<uintptr_t>(a.ptr);
  if (p % static_cast<uintptr_t>(a.esize) != 0)
    return fail(RLCA_EINVAL, "%s is not aligned to its element size (%lld bytes)", a.name,
                static_cast<long long>(a.esize));
  if (a.ld < a.width)
    return fail(RLCA_EINVAL, "ld_%s = %lld is smaller than the row length %lld", a.name,
                static_cast<long long>(a.ld), static_cast<long long>(a.width));
  if (a.ld > INT32_MAX && !a.one_row)
    return fail(RLCA_EINVAL, "ld_%s = %lld exceeds 2^31-1", a.name, static_cast<long long>(a.ld));
  // Span in elements: (N-1)*ld + width, checked against overflow.
  const int64_t lim = INT64_MAX / a.esize;
  if (N > 1 && a.ld > (lim - a.width) / (N - 1))
    return fail(RLCA_EINVAL, "%s: %lld rows of stride %lld overflow the address space", a.name,
                static_cast<long long>(N), static_cast<long long>(a.ld));
  const int64_t elems = (N - 1) * a.ld + a.width;
  a.lo = p;
  a.hi = p + static_cast<uintptr_t>(elems * a.esize);
  if (a.hi < a.lo) return fail(RLCA_EINVAL, "%s: address range wraps around", a.name);
  return RLCA_OK;
}

int check_aliasing(Arr *arrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!arrs[i].output || arrs[i].ptr == nullptr) continue;
    for (int j = 0; j < n; ++j) {
      if (i == j || arrs[j].ptr == nullptr) continue;
      if (arrs[j].output && j < i) continue;  // each output pair once
      if (arrs[i].lo < arrs[j].hi && arrs[j].lo < arrs[i].hi)
        return fail(RLCA_EALIAS, "output %s overlaps %s %s", arrs[i].name,
                    arrs[j].output ? "output" : "input", arrs[j].name);
    }
  }
  return RLCA_OK;
}

int check_unit(const char *name, float x) {
  if (!(x >= 0.f && x <= 1.f)) return fail(RLCA_EINVAL, "%s = %g must lie in [0, 1]", name, x);
  return RLCA_OK;
}

int check_clip(const char *name, float x) {
  if (!(x > 0.f)) return fail(RLCA_EINVAL, "%s = %g must be > 0", name, x);
  return RLCA_OK;
}

int check_sizes(int64_t N, int64_t T, int dtype) {
  if (N < 0 || T < 0)
    return fail(RLCA_EINVAL, "num_envs = %lld and T = %lld must be >= 0",
                static_cast<long long>(N), static_cast<long long>(T));
  if (N > INT32_MAX) return fail(RLCA_EINVAL, "num_envs = %lld exceeds 2^31-1", static_cast<long long>(N));
  if (T > INT32_MAX - 1)
    return fail(RLCA_EINVAL, "T = %lld exceeds 2^31-2", static_cast<long long>(T));
  if (dtype != RLCA_F32 && dtype != RLCA_BF16) return fail(RLCA_EDTYPE, "unknown dtype %d", dtype);
  return RLCA_OK;
}

#define RLCA_TRY(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != RLCA_OK) return rc_; \
  } while (0)

int launch(int algo, int dtype, const Args &args, void *stream) {
  const int v = t_forced_variant >= 0 ? t_forced_variant : auto_variant(args.N, args.T, dtype);
  const Variant var = kVariants[v];
  dim3 grid, block;
  if (var.WPR > 1) {
    grid = dim3(static_cast<unsigned>(args.N));
    block = dim3(64 * var.WPR);
  } else {
    const int64_t rows_per_wg = 4 * (64 / var.LPR);
    grid = dim3(static_cast<unsigned>((args.N + rows_per_wg - 1) / rows_per_wg));
    block = dim3(256);
  }
  Args a = args;
  // Hot streams (see scan_kernels.hpp), passed again as preloaded scalars.
  const void *hot[5] = {a.r, nullptr, nullptr, nullptr, nullptr};
  int64_t hld[5] = {a.ld_r, 0, 0, 0, 0};  // stride of each hot [N,T] stream (0: none)
  int64_t ldx = 0;
  switch (algo) {
    case kReturns:
      hot[1] = a.term; hld[1] = a.ld_term;
      hot[2] = a.trunc; hld[2] = a.ld_trunc;
      hot[3] = a.tv; hld[3] = a.ld_tv;
      hot[4] = a.boot;  // a [N] vector: no stride
      break;
    case kGae:
    case kTdLambda:
      hot[1] = a.v; ldx = a.ld_v;
      hot[2] = a.term; hld[2] = a.ld_term;
      hot[3] = a.trunc; hld[3] = a.ld_trunc;
      hot[4] = a.tv; hld[4] = a.ld_tv;
      break;
    case kVtrace:
      hot[1] = a.v; ldx = a.ld_v;
      hot[2] = a.lr; hld[2] = a.ld_lr;
      hot[3] = a.term; hld[3] = a.ld_term;
      hot[4] = a.trunc; hld[4] = a.ld_trunc;
      break;
    case kRetrace:
      hot[1] = a.v; hld[1] = a.ld_v;
      hot[2] = a.eq; hld[2] = a.ld_eq;
      hot[3] = a.lr; hld[3] = a.ld_lr;
      hot[4] = a.term; hld[4] = a.ld_term;
      ldx = a.trunc != nullptr ? 1 : 0;
      break;
    default:  // kEligibility, kCumsum
      hot[1] = a.term; hld[1] = a.ld_term;
      hot[2] = a.trunc; hld[2] = a.ld_trunc;
      hot[3] = a.boot;  // initial carry, a [N] vector: no stride
      break;
  }
  bool uniform = true;
  for (int i = 1; i < 5; ++i)
    if (hot[i] != nullptr && hld[i] != 0 && hld[i] != a.ld_r) uniform = false;
  int N32 = static_cast<int>(a.N);
  int T32 = static_cast<int>(a.T);
  int ldT = static_cast<int>(a.ld_r);
  int ldX = static_cast<int>(ldx);
  void *kargs[] = {&hot[0], &hot[1], &hot[2], &hot[3], &hot[4], &N32, &T32, &ldT, &ldX, &a};
  const hipError_t e = hipLaunchKernel(kernel_for(algo, dtype, v, uniform), grid, block, kargs, 0,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RLCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  t_last_variant = v;
  return RLCA_OK;
}

int64_t esize_of(int dtype) { return dtype == RLCA_BF16 ? 2 : 4; }

}  // namespace
}  // namespace rlca

using namespace rlca;

extern "C" {

int rlca_returns(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                 const void *bootstrap, float gamma, float *returns, int64_t ld_returns,
                 void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {"bootstrap", bootstrap, num_envs, num_envs, es, false, false, true},
      {"returns", returns, ld_returns, T, 4, true, true},
  };
  if (num_envs == 0 || T == 0) return RLCA_OK;
  for (Arr &a : arrs) RLCA_TRY(check_array(a, num_envs));
  RLCA_TRY(check_aliasing(arrs, 6));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.boot = bootstrap;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = returns; a.ld_o0 = ld_returns;
  a.gamma = gamma; a.lam = 1.f; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return launch(kReturns, dtype, a, stream);
}

static int gae_like(int algo, int64_t num_envs, int64_t T, int dtype, const void *rewards,
                    int64_t ld_rewards, const void *values, int64_t ld_values,
                    const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                    int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                    float gamma, float lam, float *out0, int64_t ld_out0, float *out1,
                    int64_t ld_out1, const char *name0, const char *name1, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"values", values, ld_values, T + 1, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {name0, out0, ld_out0, T, 4, true, true},
      {name1, out1, ld_out1, T, 4, false, true},
  };
  if (num_envs == 0 || T == 0) return RLCA_OK;
  for (Arr &a : arrs) RLCA_TRY(check_array(a, num_envs));
  RLCA_TRY(check_aliasing(arrs, 7));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = values; a.ld_v = ld_values;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = out0; a.ld_o0 = ld_out0;
  a.o1 = out1; a.ld_o1 = ld_out1;
  a.gamma = gamma; a.lam = lam; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return launch(algo, dtype, a, stream);
}

int rlca_gae(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
             const void *values, int64_t ld_values, const uint8_t *terminated,
             int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
             const void *trunc_values, int64_t ld_trunc_values, float gamma, float lam,
             float *advantages, int64_t ld_advantages, float *targets, int64_t ld_targets,
             void *stream) {
  return gae_like(kGae, num_envs, T, dtype, rewards, ld_rewards, values, ld_values, terminated,
                  ld_terminated, truncated, ld_truncated, trunc_values, ld_trunc_values, gamma,
                  lam, advantages, ld_advantages, targets, ld_targets, "advantages", "targets",
                  stream);
}

int rlca_td_lambda(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                   int64_t ld_rewards, const void *values, int64_t ld_values,
                   const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                   int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                   float gamma, float lam, float *lambda_returns, int64_t ld_lambda_returns,
                   void *stream) {
  return gae_like(kTdLambda, num_envs, T, dtype, rewards, ld_rewards, values, ld_values,
                  terminated, ld_terminated, truncated, ld_truncated, trunc_values,
                  ld_trunc_values, gamma, lam, lambda_returns, ld_lambda_returns, nullptr, 0,
                  "lambda_returns", "unused", stream);
}

int rlca_vtrace(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                const void *values, int64_t ld_values, const void *log_rhos,
                int64_t ld_log_rhos, const uint8_t *terminated, int64_t ld_terminated,
                const uint8_t *truncated, int64_t ld_truncated, const void *trunc_values,
                int64_t ld_trunc_values, float gamma, float lam, float rho_bar, float c_bar,
                float pg_rho_bar, float *vs, int64_t ld_vs, float *pg_advantages,
                int64_t ld_pg_advantages, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("rho_bar", rho_bar));
  RLCA_TRY(check_clip("c_bar", c_bar));
  RLCA_TRY(check_clip("pg_rho_bar", pg_rho_bar));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"values", values, ld_values, T + 1, es, true, false},
      {"log_rhos", log_rhos, ld_log_rhos, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {"vs", vs, ld_vs, T, 4, true, true},
      {"pg_advantages", pg_advantages, ld_pg_advantages, T, 4, false, true},
  };
  if (num_envs == 0 || T == 0) return RLCA_OK;
  for (Arr &a : arrs) RLCA_TRY(check_array(a, num_envs));
  RLCA_TRY(check_aliasing(arrs, 8));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = values; a.ld_v = ld_values;
  a.lr = log_rhos; a.ld_lr = ld_log_rhos;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = vs; a.ld_o0 = ld_vs;
  a.o1 = pg_advantages; a.ld_o1 = ld_pg_advantages;
  a.gamma = gamma; a.lam = lam; a.rho_bar = rho_bar; a.c_bar = c_bar; a.pg_rho_bar = pg_rho_bar;
  return launch(kVtrace, dtype, a, stream);
}

int rlca_retrace(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const void *q_taken, int64_t ld_q_taken, const void *exp_q_next,
                 int64_t ld_exp_q_next, const void *log_rhos, int64_t ld_log_rhos,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, float gamma, float lam, float c_bar, float *q_ret,
                 int64_t ld_q_ret, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("c_bar", c_bar));
  const int64_t es = esize_of(dtype);
  Arr arrs[] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"q_taken", q_taken, ld_q_taken, T, es, true, false},
      {"exp_q_next", exp_q_next, ld_exp_q_next, T, es, true, false},
      {"log_rhos", log_rhos, ld_log_rhos, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"q_ret", q_ret, ld_q_ret, T, 4, true, true},
  };
  if (num_envs == 0 || T == 0) return RLCA_OK;
  for (Arr &a : arrs) RLCA_TRY(check_array(a, num_envs));
  RLCA_TRY(check_aliasing(arrs, 7));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = q_taken; a.ld_v = ld_q_taken;
  a.eq = exp_q_next; a.ld_eq = ld_exp_q_next;
  a.lr = log_rhos; a.ld_lr = ld_log_rhos;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = q_ret; a.ld_o0 = ld_q_ret;
  a.gamma = gamma; a.lam = lam; a.rho_bar = 1.f; a.c_bar = c_bar; a.pg_rho_bar = 1.f;
  return launch(kRetrace, dtype, a, stream);
}

static int forward_like(int algo, int64_t num_envs, int64_t T, int dtype, const void *x,
                        int64_t ld_x, const uint8_t *terminated, int64_t ld_terminated,
                        const uint8_t *truncated, int64_t ld_truncated, const void *init,
                        float gamma, float lam, float *out, int64_t ld_out, const char *init_name,
                        const char *out_name, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  const int64_t es = esize_of(dtype);
  Arr arrs[] = {
      {"x", x, ld_x, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {init_name, init, num_envs, num_envs, es, false, false, true},
      {out_name, out, ld_out, T, 4, true, true},
  };
  if (num_envs == 0 || T == 0) return RLCA_OK;
  for (Arr &a : arrs) RLCA_TRY(check_array(a, num_envs));
  RLCA_TRY(check_aliasing(arrs, 5));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = x; a.ld_r = ld_x;
  a.boot = init;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = out; a.ld_o0 = ld_out;
  a.gamma = gamma; a.lam = lam; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return launch(algo, dtype, a, stream);
}

int rlca_eligibility_trace(int64_t num_envs, int64_t T, int dtype, const void *x, int64_t ld_x,
                           const uint8_t *terminated, int64_t ld_terminated,
                           const uint8_t *truncated, int64_t ld_truncated, const void *z_init,
                           float gamma, float lam, float *traces, int64_t ld_traces,
                           void *stream) {
  return forward_like(kEligibility, num_envs, T, dtype, x, ld_x, terminated, ld_terminated,
                      truncated, ld_truncated, z_init, gamma, lam, traces, ld_traces, "z_init",
                      "traces", stream);
}

int rlca_episodic_cumsum(int64_t num_envs, int64_t T, int dtype, const void *x, int64_t ld_x,
                         const uint8_t *terminated, int64_t ld_terminated,
                         const uint8_t *truncated, int64_t ld_truncated, const void *s_init,
                         float *sums, int64_t ld_sums, void *stream) {
  return forward_like(kCumsum, num_envs, T, dtype, x, ld_x, terminated, ld_terminated, truncated,
                      ld_truncated, s_init, 1.f, 1.f, sums, ld_sums, "s_init", "sums", stream);
}

const char *rlca_last_error(void) { return t_last_error.c_str(); }

int rlca_version(void) { return 100; }  // 0.1.0

int rlca_num_variants(void) { return kNumVariants; }

int rlca_set_variant(int variant) {
  if (variant < -1 || variant >= kNumVariants) return -2;
  const int prev = t_forced_variant;
  t_forced_variant = variant;
  return prev;
}

int rlca_variant_info(int variant, int dtype, int *steps_per_lane_out, int *lanes_per_row,
                      int *waves_per_row) {
  if (variant < 0 || variant >= kNumVariants)
    return fail(RLCA_EINVAL, "unknown variant %d", variant);
  if (dtype != RLCA_F32 && dtype != RLCA_BF16) return fail(RLCA_EDTYPE, "unknown dtype %d", dtype);
  const Variant v = kVariants[variant];
  if (steps_per_lane_out) *steps_per_lane_out = kStepsPerLane;
  if (lanes_per_row) *lanes_per_row = v.WPR > 1 ? 64 * v.WPR : v.LPR;
  if (waves_per_row) *waves_per_row = v.WPR;
  return RLCA_OK;
}

int rlca_last_variant(void) { return t_last_variant; }

}  // extern "C"
