// kernels_chain.hip -- the chained instances (one-launch split calls).
#include "kernel_table.hpp"

namespace rlca {

const void *chain_kernel(int algo, int dtype, int v, int tiles) {
  switch (algo) {
    case kReturns: return chain_ptr<kReturns>(dtype, v, tiles);
    case kGae: return chain_ptr<kGae>(dtype, v, tiles);
    case kTdLambda: return chain_ptr<kTdLambda>(dtype, v, tiles);
    case kVtrace: return chain_ptr<kVtrace>(dtype, v, tiles);
    case kRetrace: return chain_ptr<kRetrace>(dtype, v, tiles);
    case kEligibility: return chain_ptr<kEligibility>(dtype, v, tiles);
    case kCumsum: return chain_ptr<kCumsum>(dtype, v, tiles);
    case kAffine: return chain_ptr<kAffine>(dtype, v, tiles);
    case kAffineFwd: return chain_ptr<kAffineFwd>(dtype, v, tiles);
    default: return nullptr;
  }
}

}  // namespace rlca
