// kernels_probs.hip -- kernel instances of the policy-table entry points.
#include "probs_kernels.hpp"
#include "rlca.h"
#include "variants.hpp"

namespace rlca {

const void *probs_kernel_for(int algo, int dtype) {
  if (algo == kRetrace)
    return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&probs_kernel<kRetrace, bf16_t>)
                              : reinterpret_cast<const void *>(&probs_kernel<kRetrace, float>);
  if (algo == kVtrace)
    return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&probs_kernel<kVtrace, bf16_t>)
                              : reinterpret_cast<const void *>(&probs_kernel<kVtrace, float>);
  return nullptr;
}

}  // namespace rlca
