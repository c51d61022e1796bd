"""MI355X (gfx950) scaled-dot-product attention: causal GQA prefill and
paged single-token decode behind the C ABI of libattn.so (include/attn.h),
with the paged KV append and the fused QK-norm + rotary step around them.

``binding`` holds the ctypes front end (same names as the C entry points);
``workloads`` the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_LAUNCH,
    ATTN_ERR_UNSUPPORTED,
    ATTN_ERR_WORKSPACE,
    ATTN_OK,
    AttnError,
    attn_abi_version,
    attn_cross_attention,
    attn_cross_attention_workspace_size,
    attn_decode_paged,
    attn_decode_paged_scratch,
    attn_decode_paged_shared_prefix,
    attn_decode_paged_shared_prefix_workspace_size,
    attn_decode_paged_workspace_size,
    attn_kv_append,
    attn_prefill,
    attn_prefill_qk_norm_rope,
    attn_qk_norm_rope,
    attn_qk_norm_rope_append,
    attn_rope_table,
    attn_status_string,
    load_library,
)
