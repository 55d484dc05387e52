// kernels_plain.hip -- the kernel instances of the plain windowed entry
// points (no carry vectors).
#include "kernel_table.hpp"

namespace rlca {

const void *plain_kernel(int algo, int dtype, int v, bool uniform, bool one) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, false>(dtype, v, uniform, one);
    case kGae: return kernel_ptr<kGae, false>(dtype, v, uniform, one);
    case kTdLambda: return kernel_ptr<kTdLambda, false>(dtype, v, uniform, one);
    case kVtrace: return kernel_ptr<kVtrace, false>(dtype, v, uniform, one);
    case kRetrace: return kernel_ptr<kRetrace, false>(dtype, v, uniform, one);
    case kEligibility: return kernel_ptr<kEligibility, false>(dtype, v, uniform, one);
    case kCumsum: return kernel_ptr<kCumsum, false>(dtype, v, uniform, one);
    default: return nullptr;
  }
}

}  // namespace rlca
