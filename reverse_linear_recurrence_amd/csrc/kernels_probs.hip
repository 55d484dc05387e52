// kernels_probs.hip -- kernel instances of the policy-table entry points.
#include "probs_kernels.hpp"
#include "rlca.h"
#include "variants.hpp"

namespace rlca {

template <int Algo, int WPR>
const void *probs_kernel_for(int dtype) {
  return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&probs_kernel<Algo, bf16_t, WPR>)
                            : reinterpret_cast<const void *>(&probs_kernel<Algo, float, WPR>);
}

const void *probs_kernel_for(int algo, int dtype, int waves_per_row) {
  const bool wide = waves_per_row > 1;
  if (algo == kRetrace)
    return wide ? probs_kernel_for<kRetrace, 4>(dtype) : probs_kernel_for<kRetrace, 1>(dtype);
  if (algo == kVtrace)
    return wide ? probs_kernel_for<kVtrace, 4>(dtype) : probs_kernel_for<kVtrace, 1>(dtype);
  return nullptr;
}

}  // namespace rlca
