// kernels_window.hip -- the kernel instances of the window entry points
// (carry vector in; carry and carry map out), including the generic scan.
#include "kernel_table.hpp"

namespace rlca {

const void *window_kernel(int algo, int dtype, int v, bool uniform) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, true>(dtype, v, uniform);
    case kGae: return kernel_ptr<kGae, true>(dtype, v, uniform);
    case kTdLambda: return kernel_ptr<kTdLambda, true>(dtype, v, uniform);
    case kVtrace: return kernel_ptr<kVtrace, true>(dtype, v, uniform);
    case kRetrace: return kernel_ptr<kRetrace, true>(dtype, v, uniform);
    case kEligibility: return kernel_ptr<kEligibility, true>(dtype, v, uniform);
    case kCumsum: return kernel_ptr<kCumsum, true>(dtype, v, uniform);
    case kAffine: return kernel_ptr<kAffine, true>(dtype, v, uniform);
    case kAffineFwd: return kernel_ptr<kAffineFwd, true>(dtype, v, uniform);
    default: return nullptr;
  }
}

}  // namespace rlca
