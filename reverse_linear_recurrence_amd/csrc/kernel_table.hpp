// kernel_table.hpp -- instantiation of scan_kernel over variants, dtypes and
// stride modes for one algorithm; included by the kernel translation units.
#pragma once

#include "rlca.h"
#include "scan_kernels.hpp"
#include "variants.hpp"

namespace rlca {

template <int A, typename InT, int V, bool U, bool C, int O, bool AL>
const void *kernel_ptr() {
  constexpr Variant v = kVariants[V];
  constexpr int K = steps_per_lane(v, sizeof(InT) == 2, A == kVtrace);
  return reinterpret_cast<const void *>(&scan_kernel<A, InT, K, v.LPR, v.WPR, U, C, O, AL>);
}

template <int A, typename InT, bool U, bool C, int O = 0, bool AL = false>
const void *kernel_ptr(int v) {
  static_assert(kNumVariants == 9, "one case per variant");
  switch (v) {
    case 0: return kernel_ptr<A, InT, 0, U, C, O, AL>();
    case 1: return kernel_ptr<A, InT, 1, U, C, O, AL>();
    case 2: return kernel_ptr<A, InT, 2, U, C, O, AL>();
    case 3: return kernel_ptr<A, InT, 3, U, C, O, AL>();
    case 4: return kernel_ptr<A, InT, 4, U, C, O, AL>();
    case 5: return kernel_ptr<A, InT, 5, U, C, O, AL>();
    case 6: return kernel_ptr<A, InT, 6, U, C, O, AL>();
    case 7: return kernel_ptr<A, InT, 7, U, C, O, AL>();
    default: return kernel_ptr<A, InT, 8, U, C, O, AL>();
  }
}

template <int A, typename InT, bool C, int O>
const void *fixed_tiles_ptr(int v, bool aligned) {
  constexpr bool kHasAligned = !Uses<A>::prev_flags;  // forward mirrors read from t - 1
  if constexpr (kHasAligned) {
    if (aligned) return kernel_ptr<A, InT, true, C, O, true>(v);
  }
  return kernel_ptr<A, InT, true, C, O, false>(v);
}

// tiles: 1 or 2 for the instances of rows of exactly one or two whole tiles
// (0: the general instance), aligned: their twins for 4-byte aligned flag
// rows (reverse recurrences and the generic scan); they exist for the plain
// and the window instances with a uniform row stride.
template <int A, bool C>
const void *kernel_ptr(int dtype, int v, bool uniform, int tiles = 0, bool aligned = false) {
  if (uniform && tiles == 1) {
    return dtype == RLCA_BF16 ? fixed_tiles_ptr<A, bf16_t, C, 1>(v, aligned)
                              : fixed_tiles_ptr<A, float, C, 1>(v, aligned);
  }
  if (uniform && tiles == 2) {
    return dtype == RLCA_BF16 ? fixed_tiles_ptr<A, bf16_t, C, 2>(v, aligned)
                              : fixed_tiles_ptr<A, float, C, 2>(v, aligned);
  }
  if (dtype == RLCA_BF16)
    return uniform ? kernel_ptr<A, bf16_t, true, C>(v) : kernel_ptr<A, bf16_t, false, C>(v);
  return uniform ? kernel_ptr<A, float, true, C>(v) : kernel_ptr<A, float, false, C>(v);
}

// Chained instances (one-launch split calls): window instances with a
// uniform row stride for segments of exactly one or two whole tiles, in the
// tilings with whole wavefronts per row (variants 3-8).
template <int A, typename InT, int V, int O>
const void *chain_ptr() {
  constexpr Variant v = kVariants[V];
  static_assert(v.WPR > 1, "chained instances need whole-wavefront rows");
  constexpr int K = steps_per_lane(v, sizeof(InT) == 2, A == kVtrace);
  return reinterpret_cast<const void *>(
      &scan_kernel<A, InT, K, v.LPR, v.WPR, true, true, O, false, true>);
}

template <int A, typename InT, int O>
const void *chain_ptr(int v) {
  switch (v) {
    case 3: return chain_ptr<A, InT, 3, O>();
    case 4: return chain_ptr<A, InT, 4, O>();
    case 5: return chain_ptr<A, InT, 5, O>();
    case 6: return chain_ptr<A, InT, 6, O>();
    case 7: return chain_ptr<A, InT, 7, O>();
    case 8: return chain_ptr<A, InT, 8, O>();
    default: return nullptr;
  }
}

template <int A>
const void *chain_ptr(int dtype, int v, int tiles) {
  if (tiles == 1) return dtype == RLCA_BF16 ? chain_ptr<A, bf16_t, 1>(v) : chain_ptr<A, float, 1>(v);
  if (tiles == 2) return dtype == RLCA_BF16 ? chain_ptr<A, bf16_t, 2>(v) : chain_ptr<A, float, 2>(v);
  return nullptr;
}

}  // namespace rlca
