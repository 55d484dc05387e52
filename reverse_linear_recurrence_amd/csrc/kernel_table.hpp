// kernel_table.hpp -- instantiation of scan_kernel over variants, dtypes and
// stride modes for one algorithm; included by the kernel translation units.
#pragma once

#include "rlca.h"
#include "scan_kernels.hpp"
#include "variants.hpp"

namespace rlca {

template <int A, typename InT, int V, bool U, bool C, bool O, bool AL>
const void *kernel_ptr() {
  constexpr Variant v = kVariants[V];
  constexpr int K = steps_per_lane(v, sizeof(InT) == 2, A == kVtrace);
  return reinterpret_cast<const void *>(&scan_kernel<A, InT, K, v.LPR, v.WPR, U, C, O, AL>);
}

template <int A, typename InT, bool U, bool C, bool O = false, bool AL = false>
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

template <int A, typename InT, bool C>
const void *one_tile_ptr(int v, bool aligned) {
  constexpr bool kHasAligned = !Uses<A>::prev_flags;  // forward mirrors read from t - 1
  if constexpr (kHasAligned) {
    if (aligned) return kernel_ptr<A, InT, true, C, true, true>(v);
  }
  return kernel_ptr<A, InT, true, C, true, false>(v);
}

// one: the one-tile instance (rows of exactly one whole tile), aligned: its
// twin for 4-byte aligned flag rows (reverse recurrences); both exist for the
// plain instances (C false) with a uniform row stride.
template <int A, bool C>
const void *kernel_ptr(int dtype, int v, bool uniform, bool one = false, bool aligned = false) {
  if constexpr (!C) {
    if (uniform && one) {
      return dtype == RLCA_BF16 ? one_tile_ptr<A, bf16_t, C>(v, aligned)
                                : one_tile_ptr<A, float, C>(v, aligned);
    }
  }
  if (dtype == RLCA_BF16)
    return uniform ? kernel_ptr<A, bf16_t, true, C, false>(v)
                   : kernel_ptr<A, bf16_t, false, C, false>(v);
  return uniform ? kernel_ptr<A, float, true, C, false>(v) : kernel_ptr<A, float, false, C, false>(v);
}

}  // namespace rlca
