// kernels_window.hip -- the kernel instances of the window entry points
// (carry vector in; carry and carry map out), including the generic scan.
#include "kernel_table.hpp"

namespace rlca {

const void *window_kernel(int algo, int dtype, int v, bool uniform, int tiles,
                          bool aligned) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, true>(dtype, v, uniform, tiles, aligned);
    case kGae: return kernel_ptr<kGae, true>(dtype, v, uniform, tiles, aligned);
    case kTdLambda: return kernel_ptr<kTdLambda, true>(dtype, v, uniform, tiles, aligned);
    case kVtrace: return kernel_ptr<kVtrace, true>(dtype, v, uniform, tiles, aligned);
    case kRetrace: return kernel_ptr<kRetrace, true>(dtype, v, uniform, tiles, aligned);
    case kEligibility: return kernel_ptr<kEligibility, true>(dtype, v, uniform, tiles, aligned);
    case kCumsum: return kernel_ptr<kCumsum, true>(dtype, v, uniform, tiles, aligned);
    case kAffine: return kernel_ptr<kAffine, true>(dtype, v, uniform, tiles, aligned);
    case kAffineFwd: return kernel_ptr<kAffineFwd, true>(dtype, v, uniform, tiles, aligned);
    default: return nullptr;
  }
}

}  // namespace rlca
