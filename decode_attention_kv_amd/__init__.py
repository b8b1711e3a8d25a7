"""Decode-phase attention over a KV cache, native to AMD MI355X (gfx950).

The product is the C-ABI library ``libdakv.so`` (declared in include/dakv.h) with
hand-written HIP kernels; ``ops`` is its thin torch-facing binding.  There is no
CPU fallback: loading fails loudly when the library has not been built.
"""

from .ops import (
    kv_append,
    kv_append_fp8,
    decode_attn_static_fp8,
    decode_step_static_fp8,
    kv_append_fp4,
    decode_attn_static_fp4,
    paged_append_fp8,
    decode_attn_paged_fp8,
    copy_kvcache,
    trim_kvcache,
    decode_attn_static,
    decode_attn_static_workspace_size,
    decode_step_static,
    gather_pa_kv_cache,
    decode_attn_paged,
    decode_attn_paged_workspace_size,
    sparse_topk_attn,
    latent_append_fp8,
    sparse_topk_attn_fp8,
    latent_append_fp4,
    sparse_topk_attn_fp4,
    sparse_topk_decode_attn,
    sparse_topk_decode_attn_workspace_size,
    validate_paged,
    validate_sparse,
    validate_range,
)
from ._lib import DakvError, lib, strerror

__all__ = [
    "kv_append",
    "kv_append_fp8",
    "decode_attn_static_fp8",
    "decode_step_static_fp8",
    "kv_append_fp4",
    "decode_attn_static_fp4",
    "paged_append_fp8",
    "decode_attn_paged_fp8",
    "copy_kvcache",
    "trim_kvcache",
    "decode_attn_static",
    "decode_attn_static_workspace_size",
    "decode_step_static",
    "gather_pa_kv_cache",
    "decode_attn_paged",
    "decode_attn_paged_workspace_size",
    "sparse_topk_attn",
    "latent_append_fp8",
    "sparse_topk_attn_fp8",
    "latent_append_fp4",
    "sparse_topk_attn_fp4",
    "sparse_topk_decode_attn",
    "sparse_topk_decode_attn_workspace_size",
    "validate_paged",
    "validate_sparse",
    "validate_range",
    "DakvError",
    "lib",
    "strerror",
]
