// kernels_materialized.hip -- kernel instances of the materialized doubling
// scan (materialized.hpp), the pages' comparison baseline re-created in HIP.
#include "materialized.hpp"
#include "rlca.h"

namespace rlca {

template <int A>
const void *coeffs_for(int dtype) {
  return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&mat_coeffs<A, bf16_t>)
                            : reinterpret_cast<const void *>(&mat_coeffs<A, float>);
}

template <int A>
const void *epilogue_for(int dtype) {
  return dtype == RLCA_BF16 ? reinterpret_cast<const void *>(&mat_epilogue<A, bf16_t>)
                            : reinterpret_cast<const void *>(&mat_epilogue<A, float>);
}

const void *mat_coeffs_kernel(int algo, int dtype) {
  switch (algo) {
    case kReturns: return coeffs_for<kReturns>(dtype);
    case kGae: return coeffs_for<kGae>(dtype);
    case kTdLambda: return coeffs_for<kTdLambda>(dtype);
    case kVtrace: return coeffs_for<kVtrace>(dtype);
    case kRetrace: return coeffs_for<kRetrace>(dtype);
    default: return nullptr;
  }
}

const void *mat_epilogue_kernel(int algo, int dtype) {
  switch (algo) {
    case kReturns: return epilogue_for<kReturns>(dtype);
    case kGae: return epilogue_for<kGae>(dtype);
    case kTdLambda: return epilogue_for<kTdLambda>(dtype);
    case kVtrace: return epilogue_for<kVtrace>(dtype);
    case kRetrace: return epilogue_for<kRetrace>(dtype);
    default: return nullptr;
  }
}

const void *mat_double_kernel() { return reinterpret_cast<const void *>(&mat_double<float>); }

}  // namespace rlca
