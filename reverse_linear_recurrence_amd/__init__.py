"""Reverse linear recurrences for RL credit assignment on AMD MI355X (gfx950).

Python binding of ``librlca.so`` (C ABI in ``include/rlca.h``).  This module
only marshals arguments: it checks shapes, dtypes and devices, allocates the
outputs with torch, and passes raw device pointers, row strides and the
current HIP stream to the library, which does every step of the computation
in its HIP kernels.  There is no fallback: if the library is missing or the
tensors are not on a GPU, the call raises.

Functions (same names as the C ABI):
    rlca_returns, rlca_gae, rlca_td_lambda, rlca_vtrace, rlca_retrace,
    rlca_eligibility_trace, rlca_episodic_cumsum,
their window forms (carry in; carry and carry map out) with the suffix
_chunk (and rlca_gae_chunk_noalloc, which needs no workspace), the generic
segmented scan rlca_affine_scan, Retrace and V-trace from
policy log-probability tables (rlca_retrace_probs, rlca_vtrace_probs), the
materialized doubling scan the pages compare against (rlca_X_materialized), and the
tiling controls rlca_set_variant, rlca_num_variants,
rlca_variant_info, rlca_last_variant, the split-call sizes
rlca_split_segments and rlca_split_workspace_bytes (split_workspace allocates
one), the split form control rlca_set_chained, rlca_last_launches,
rlca_last_segments, plus
rlca_version.
"""
from ._binding import (  # noqa: F401
    ALGO_CODES,
    RLCA_BF16,
    RLCA_EALIAS,
    RLCA_EDTYPE,
    RLCA_EHIP,
    RLCA_EINVAL,
    RLCA_F32,
    RLCA_OK,
    RlcaError,
    TIMED_LIB_PATH,
    lib_path,
    load_library,
    rlca_affine_scan,
    rlca_eligibility_trace,
    rlca_eligibility_trace_chunk,
    rlca_episodic_cumsum,
    rlca_episodic_cumsum_chunk,
    rlca_gae,
    rlca_gae_chunk,
    rlca_gae_chunk_noalloc,
    rlca_gae_materialized,
    rlca_last_launches,
    rlca_last_segments,
    rlca_last_variant,
    rlca_materialized_workspace_bytes,
    rlca_num_variants,
    rlca_retrace,
    rlca_retrace_chunk,
    rlca_retrace_materialized,
    rlca_retrace_probs,
    rlca_retrace_probs_chunk,
    rlca_returns,
    rlca_returns_chunk,
    rlca_returns_materialized,
    rlca_set_chained,
    rlca_set_variant,
    rlca_split_segments,
    rlca_split_workspace_bytes,
    rlca_td_lambda,
    rlca_td_lambda_chunk,
    rlca_td_lambda_materialized,
    rlca_timestamps,
    rlca_variant_info,
    rlca_version,
    rlca_vtrace,
    rlca_vtrace_chunk,
    rlca_vtrace_materialized,
    rlca_vtrace_probs,
    rlca_vtrace_probs_chunk,
    split_workspace,
    use_library,
)
