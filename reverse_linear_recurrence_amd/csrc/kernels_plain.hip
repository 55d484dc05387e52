// kernels_plain.hip -- the kernel instances of the plain windowed entry
// points (no carry vectors).
#include "kernel_table.hpp"

namespace rlca {

const void *plain_kernel(int algo, int dtype, int v, bool uniform) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, false>(dtype, v, uniform);
    case kGae: return kernel_ptr<kGae, false>(dtype, v, uniform);
    case kTdLambda: return kernel_ptr<kTdLambda, false>(dtype, v, uniform);
    case kVtrace: return kernel_ptr<kVtrace, false>(dtype, v, uniform);
    case kRetrace: return kernel_ptr<kRetrace, false>(dtype, v, uniform);
    case kEligibility: return kernel_ptr<kEligibility, false>(dtype, v, uniform);
    case kCumsum: return kernel_ptr<kCumsum, false>(dtype, v, uniform);
    default: return nullptr;
  }
}

}  // namespace rlca
