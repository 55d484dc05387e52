// kernels_plain.hip -- the kernel instances of the plain windowed entry
// points (no carry vectors).
#include "kernel_table.hpp"

namespace rlca {

const void *plain_kernel(int algo, int dtype, int v, bool uniform, int tiles,
                          bool aligned) {
  switch (algo) {
    case kReturns: return kernel_ptr<kReturns, false>(dtype, v, uniform, tiles, aligned);
    case kGae: return kernel_ptr<kGae, false>(dtype, v, uniform, tiles, aligned);
    case kTdLambda: return kernel_ptr<kTdLambda, false>(dtype, v, uniform, tiles, aligned);
    case kVtrace: return kernel_ptr<kVtrace, false>(dtype, v, uniform, tiles, aligned);
    case kRetrace: return kernel_ptr<kRetrace, false>(dtype, v, uniform, tiles, aligned);
    case kEligibility: return kernel_ptr<kEligibility, false>(dtype, v, uniform, tiles, aligned);
    case kCumsum: return kernel_ptr<kCumsum, false>(dtype, v, uniform, tiles, aligned);
    default: return nullptr;
  }
}

}  // namespace rlca
