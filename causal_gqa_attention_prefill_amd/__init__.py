"""Chunked causal grouped-query prefill attention for MI355X (gfx950).

The work runs in ``libprefill_attn.so`` (HIP kernels behind the C ABI of
``include/prefill_attn.h``); ``binding`` marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    PA_DTYPE_BF16, PA_DTYPE_F16, PA_DTYPE_F32, PA_ERR_HIP, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED,
    PA_ERR_WORKSPACE, PA_OK, PrefillAttnError, PreparedCall, header_define, header_functions, library_path,
    load, plan, prefill_attn, prefill_attn_ex, prefill_attn_noalloc_ex, prefill_attn_paged_ex, prefill_attn_ring_ex,
    prefill_attn_vmirror_ex, prefill_kv_write, strerror, vmirror_bytes, workspace_bytes,
)
