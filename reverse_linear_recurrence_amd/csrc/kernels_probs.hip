// kernels_probs.hip -- kernel instances of the policy-table entry points.
#include "probs_kernels.hpp"
#include "rlca.h"
#include "variants.hpp"

namespace rlca {

template <int Algo, int WPR, bool C>
const void *probs_kernel_for(int dtype) {
  return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&probs_kernel<Algo, bf16_t, WPR, C>)
                            : reinterpret_cast<const void *>(&probs_kernel<Algo, float, WPR, C>);
}

template <int Algo, bool C>
const void *probs_kernel_for(int dtype, int waves_per_row) {
  return waves_per_row > 1 ? probs_kernel_for<Algo, 4, C>(dtype)
                           : probs_kernel_for<Algo, 1, C>(dtype);
}

const void *probs_kernel_for(int algo, int dtype, int waves_per_row, bool window) {
  if (algo == kRetrace)
    return window ? probs_kernel_for<kRetrace, true>(dtype, waves_per_row)
                  : probs_kernel_for<kRetrace, false>(dtype, waves_per_row);
  if (algo == kVtrace)
    return window ? probs_kernel_for<kVtrace, true>(dtype, waves_per_row)
                  : probs_kernel_for<kVtrace, false>(dtype, waves_per_row);
  return nullptr;
}

}  // namespace rlca
