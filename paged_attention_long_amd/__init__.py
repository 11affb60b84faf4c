"""MI355X-native paged attention of a few new query rows against a long,
growing, paged KV cache (decode, speculative verification, chunked prefill).

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI in
include/paged_attn.h (libpaged_attn.so); this package only binds it.
"""
from .binding import (  # noqa: F401
    PA_DTYPE_BF16,
    PA_DTYPE_F16,
    PA_DTYPE_FP8_E4M3,
    PA_DTYPE_INT8,
    PA_PATH_AUTO,
    PA_PATH_MFMA,
    PA_PATH_VALU,
    Handle,
    PagedAttnError,
    cache_layout,
    header_functions,
    load_library,
    make_config,
    paged_attn_create,
    paged_attn_debug_gather,
    paged_attn_debug_status,
    paged_attn_append,
    paged_attn_destroy,
    paged_attn_forward,
    paged_attn_forward_noalloc,
    paged_attn_last_error,
    paged_attn_set_tuning,
    paged_attn_version,
)
