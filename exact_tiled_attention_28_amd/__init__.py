"""Exact tiled attention (FlashAttention-2 order) for AMD MI355X / gfx950.

The computation lives in libfa.so (C ABI, include/fa.h); this package holds
the ctypes binding, the seeded input generator, the workload table and the
build script.
"""

from .binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARGUMENT,
    FA_ERR_UNSUPPORTED,
    FA_OK,
    FAError,
    backward,
    backward_varlen,
    fa_bwd,
    fa_bwd_atomic,
    fa_bwd_varlen,
    fa_bwd_workspace_bytes,
    fa_fp8_scales_count,
    fa_fwd,
    fa_fwd_fp8,
    fa_fwd_persistent,
    fa_fwd_persistent_sched_bytes,
    fa_fwd_varlen,
    fa_last_error,
    fa_quantize_fp8,
    fa_status_string,
    fa_version,
    forward,
    forward_fp8,
    forward_persistent,
    forward_varlen,
    load_library,
    new_sched,
    quantize_fp8,
)
