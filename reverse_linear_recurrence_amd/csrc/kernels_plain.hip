// kernels_plain.hip -- the kernel instances of the plain windowed entry
// points (no carry vectors).
#include "kernel_table.hpp"

namespace rlca {

const void *plain_kernel(int algo, int dtype, int v, bool uniform, bool one,
                          bool aligned) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, false>(dtype, v, uniform, one, aligned);
    case kGae: return kernel_ptr<kGae, false>(dtype, v, uniform, one, aligned);
    case kTdLambda: return kernel_ptr<kTdLambda, false>(dtype, v, uniform, one, aligned);
    case kVtrace: return kernel_ptr<kVtrace, false>(dtype, v, uniform, one, aligned);
    case kRetrace: return kernel_ptr<kRetrace, false>(dtype, v, uniform, one, aligned);
    case kEligibility: return kernel_ptr<kEligibility, false>(dtype, v, uniform, one, aligned);
    case kCumsum: return kernel_ptr<kCumsum, false>(dtype, v, uniform, one, aligned);
    default: return nullptr;
  }
}

}  // namespace rlca
