"""paged_kv_token_amd: generalized paged attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpensieve.so`` (HIP kernels behind the C ABI of
``include/pensieve.h``); this package holds its sources, the build script
and a thin ctypes binding with the same entry-point names.
"""

from .binding import (  # noqa: F401
    CONVERSATION_DTYPE,
    BatchDesc,
    PensieveError,
    PENSIEVE_BF16,
    PENSIEVE_ERR_INVALID_ARG,
    PENSIEVE_ERR_UNSUPPORTED,
    PENSIEVE_F16,
    PENSIEVE_F32,
    PENSIEVE_FP8_E4M3,
    PENSIEVE_FLAG_NO_SPLIT,
    PENSIEVE_FLAG_SINGLE_STREAM,
    PENSIEVE_FLAG_VECTOR_ONLY,
    dtype_code,
    load_library,
    conversations,
    make_desc,
    pensieve_attn_fwd,
    pensieve_attn_fwd_noalloc,
    pensieve_attn_split_merge,
    pensieve_attn_split_partial,
    pensieve_attn_workspace_size,
    pensieve_cache_build_batch,
    pensieve_cache_plan_evictions,
    pensieve_debug_plan,
    pensieve_kv_append,
    pensieve_kv_append_fp8,
    pensieve_kv_swap_in,
    pensieve_kv_swap_out,
    pensieve_trace_enable,
    pensieve_trace_read,
    pensieve_version,
)
