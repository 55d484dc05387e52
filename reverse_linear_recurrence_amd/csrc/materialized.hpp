// materialized.hpp -- the materialized O(log T) doubling scan: the baseline
// the rl-triton explainer pages measure their fused kernels against
// (Technical summary, Problem: a vectorized scan in O(log T) steps that
// writes its intermediates to HBM and reads them back at every step; Method
// 2 and Results compare the fused single pass with it).  Re-created here in
// HIP for MI355X, so that the comparison can be made on this machine.  It
// computes the same results as the fused entry points (up to rounding
// order), in 2 + ceil(log2 T) launches that each stream whole [N, T] arrays
// through HBM:
//   1. mat_coeffs: the affine pair (alpha_t, beta_t) of every step (Method
//      1; the coefficient table of the fused kernels, with the boundary
//      masks of Method 3), written to HBM;
//   2. mat_double, once per offset s = 1, 2, 4, ... < T: every step composes
//      its pair with the pair s steps later (Method 1's operator),
//        (a_t, b_t) <- (a_t + b_t a_{t+s}, b_t b_{t+s})   if t + s < T,
//      reading one pair of arrays and writing the other (Hillis-Steele), so
//      that after the last pass (a_t, b_t) composes steps t .. T-1;
//   3. mat_epilogue: A_t = a_t + b_t A_T (A_T: the per-row bootstrap of
//      discounted returns, else 0) and the algorithm's outputs from A.
// Every kernel is elementwise: one thread per step, the rows of a [N, T]
// array in blockIdx.y (strided over rows past the grid), coalesced along T.
// The pairs live in a caller workspace of 4 N T floats (two pairs of [N, T]
// arrays, row length T).
#pragma once

#include "scan_kernels.hpp"

namespace rlca {

constexpr int kMatBlock = 256;
constexpr int64_t kMatMaxGridRows = 65535;

template <typename InT>
__device__ __forceinline__ float mat_ld(const void *base, int64_t row, int64_t ld, int64_t t) {
  return Bits<InT>::to_float(Bits<InT>::load(static_cast<const InT *>(base) + row * ld + t));
}

__device__ __forceinline__ bool mat_flag(const uint8_t *base, int64_t row, int64_t ld, int64_t t) {
  return base != nullptr && base[row * ld + t] != 0;
}

// 1. (alpha_t, beta_t) per step: the coefficients of the fused kernels.  The
// arrays are read as a vectorized implementation reads them: whole, the
// truncation bootstraps included (selected away where unused).
template <int A, typename InT>
__global__ void __launch_bounds__(kMatBlock)
mat_coeffs(const Args p, float *__restrict__ alpha, float *__restrict__ beta) {
  const int64_t T = p.T;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMatBlock + threadIdx.x;
  if (t >= T) return;
  for (int64_t n = blockIdx.y; n < p.N; n += gridDim.y) {
    const bool te = mat_flag(p.term, n, p.ld_term, t);
    const bool tr = mat_flag(p.trunc, n, p.ld_trunc, t);
    const bool done = te || tr;
    const float r = mat_ld<InT>(p.r, n, p.ld_r, t);
    float a, b;
    if constexpr (A == kReturns) {
      const float tv = p.tv != nullptr ? mat_ld<InT>(p.tv, n, p.ld_tv, t) : 0.f;
      a = (tr && !te) ? fmaf(p.gamma, tv, r) : r;
      b = done ? 0.f : p.gamma;
    } else if constexpr (A == kRetrace) {
      // alpha: r + gamma (1 - term) EQ - Q; beta: gamma c_{t+1}, 0 at T-1
      const float q = mat_ld<InT>(p.v, n, p.ld_v, t);
      const float eq = mat_ld<InT>(p.eq, n, p.ld_eq, t);
      a = (te ? r : fmaf(p.gamma, eq, r)) - q;
      const float lr1 = t + 1 < T ? mat_ld<InT>(p.lr, n, p.ld_lr, t + 1) : 0.f;
      b = (done || t + 1 >= T) ? 0.f : p.gamma * (p.lam * fminf(p.c_bar, __expf(lr1)));
    } else {  // kGae, kTdLambda, kVtrace: delta_t with the successor value
      const float v = mat_ld<InT>(p.v, n, p.ld_v, t);
      const float v1 = mat_ld<InT>(p.v, n, p.ld_v, t + 1);
      const float tv = p.tv != nullptr ? mat_ld<InT>(p.tv, n, p.ld_tv, t) : 0.f;
      const float nv = te ? 0.f : (tr ? tv : v1);
      const float delta = fmaf(p.gamma, nv, r) - v;
      if constexpr (A == kVtrace) {
        const float e = __expf(mat_ld<InT>(p.lr, n, p.ld_lr, t));
        a = fminf(p.rho_bar, e) * delta;
        b = done ? 0.f : p.gamma * (p.lam * fminf(p.c_bar, e));
      } else {
        a = delta;
        b = done ? 0.f : p.gamma * p.lam;
      }
    }
    alpha[n * T + t] = a;
    beta[n * T + t] = b;
  }
}

// 2. One doubling pass: compose each step's pair with the pair s steps later
// (the later map applied first), from (a_in, b_in) into (a_out, b_out).
// (A template only so that the header defines no kernel by itself; F is
// float.)
template <typename F>
__global__ void __launch_bounds__(kMatBlock)
mat_double(const F *__restrict__ a_in, const F *__restrict__ b_in, F *__restrict__ a_out,
           F *__restrict__ b_out, int64_t N, int64_t T, int64_t s) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMatBlock + threadIdx.x;
  if (t >= T) return;
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    const int64_t i = n * T + t;
    F a = a_in[i], b = b_in[i];
    if (t + s < T) {
      a = fmaf(b, a_in[i + s], a);
      b = b * b_in[i + s];
    }
    a_out[i] = a;
    b_out[i] = b;
  }
}

// 3. A_t from the composed pairs and the row's carry, then the outputs (the
// fused kernels' epilogue).
template <int A, typename InT>
__global__ void __launch_bounds__(kMatBlock)
mat_epilogue(const Args p, const float *__restrict__ alpha, const float *__restrict__ beta) {
  const int64_t T = p.T;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMatBlock + threadIdx.x;
  if (t >= T) return;
  for (int64_t n = blockIdx.y; n < p.N; n += gridDim.y) {
    const int64_t i = n * T + t;
    float carry = 0.f;
    if constexpr (A == kReturns) {
      if (p.boot != nullptr) carry = Bits<InT>::to_float(Bits<InT>::load(
          static_cast<const InT *>(p.boot) + n));
    }
    const float x = fmaf(beta[i], carry, alpha[i]);
    float *o0 = p.o0 + n * p.ld_o0 + t;
    if constexpr (A == kReturns) {
      *o0 = x;
    } else if constexpr (A == kGae) {
      *o0 = x;
      if (p.o1 != nullptr) p.o1[n * p.ld_o1 + t] = x + mat_ld<InT>(p.v, n, p.ld_v, t);
    } else if constexpr (A == kTdLambda) {
      *o0 = x + mat_ld<InT>(p.v, n, p.ld_v, t);
    } else if constexpr (A == kRetrace) {
      *o0 = mat_ld<InT>(p.v, n, p.ld_v, t) + x;
    } else {  // kVtrace: vs and the policy-gradient advantage
      const float v = mat_ld<InT>(p.v, n, p.ld_v, t);
      *o0 = v + x;
      if (p.o1 != nullptr) {
        const bool te = mat_flag(p.term, n, p.ld_term, t);
        const bool tr = mat_flag(p.trunc, n, p.ld_trunc, t);
        const float v1 = mat_ld<InT>(p.v, n, p.ld_v, t + 1);
        const float vs1 = t + 1 < T ? v1 + alpha[i + 1] : v1;  // vs_{t+1}; V_T at T-1
        const float tv = p.tv != nullptr ? mat_ld<InT>(p.tv, n, p.ld_tv, t) : 0.f;
        const float nvs = te ? 0.f : (tr ? tv : vs1);
        const float e = __expf(mat_ld<InT>(p.lr, n, p.ld_lr, t));
        const float r = mat_ld<InT>(p.r, n, p.ld_r, t);
        p.o1[n * p.ld_o1 + t] = fminf(p.pg_rho_bar, e) * (fmaf(p.gamma, nvs, r) - v);
      }
    }
  }
}

// Host-side kernel addresses (kernels_materialized.hip).
const void *mat_coeffs_kernel(int algo, int dtype);
const void *mat_epilogue_kernel(int algo, int dtype);
const void *mat_double_kernel();

}  // namespace rlca
