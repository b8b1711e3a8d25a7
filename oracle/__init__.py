"""Plain, slow, fp64 CPU oracle for decode-phase attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library and its
Python binding) imports, calls or links this package; only the tests, the
``smoke()`` check and the CPU-baseline leg of the benchmark do.  The oracle shares
no code, tables or helpers with the HIP path.

Every function is written straight from the definitions on the source pages, in
float64, with no tiling, no splitting and no online softmax:

* ``static_cache``  -- the static preallocated buffer ``[batch, heads, capacity,
  head_dim]``, its 0/1 attention mask, append-at-write-position and masked
  scaled-dot-product decode attention (OpenVINO NPU LLM article, Part 1
  "Solution: preallocation + attention mask"; Part 2 KV-cache update;
  "Attention on the NPU" -> "incremental SDPA"), and the prefill -> generate
  copy of the cache and its roll-back (Part 2 generate flow; deployment features
  and "Current limitations").
* ``paged``         -- paged KV cache addressed through block tables: host
  validation, the ``gather_pa_kv_cache`` mapping, and paged GQA decode attention
  (PyPTO GatherPaKvCache article, section 3 "tensor contract and data
  semantics").
* ``sparse``        -- top-k sparse MLA-style decode (FlashMLA on Huawei Ascend,
  "Mathematical formulation").
* ``fp8``           -- the FP8 KV cache for decode: E4M3 codes with a power-of-two
  scale per cached row, its quantisation and the decode attention over it
  (FlashMLA on Huawei Ascend: FP8 KV read and dequantised at decode time; a
  token's values and scale kept together); also the FP8 paged pool and the FP8
  latent cache of the sparse kernel.
* ``fp4``           -- the FP4 KV cache for decode: E2M1 codes, two per byte, with
  a power-of-two scale per cached row, its quantisation and the decode attention
  over it (same page: the decode kernel reads FP8 or FP4 and dequantises it);
  also the FP4 paged pool and the FP4 latent cache of the sparse kernel.

bf16 tensors enter the oracle as their raw 16-bit patterns (``numpy.uint16``) and
are widened exactly to float64 (``bf16.widen``); copies (append, gather) move the
16-bit patterns untouched, so they can be compared bit for bit.

Parity status of each function (what pins it, from tests/test_oracle_*.py):
every function here is pinned by closed forms, printed values, invariants,
library-routine special cases or brute force; none is "parity unpinned".
"""

from .bf16 import widen, round_to_bf16_bits
from .static_cache import kv_append, decode_static, copy_kvcache, trim_kvcache
from .paged import (
    PagedIndexError,
    validate_paged,
    gather_pa_kv_cache,
    decode_paged,
    decode_paged_via_gather,
)
from .sparse import sparse_topk_attn, sparse_topk_decode, validate_sparse
from .fp8 import (
    e4m3_decode,
    e4m3_encode,
    scale_exponent,
    quantize_rows,
    kv_append_fp8,
    decode_static_fp8,
    decode_paged_fp8,
    paged_append_fp8,
    latent_append_fp8,
    sparse_topk_attn_fp8,
)
from . import fp4
from .fp4 import (
    kv_append_fp4,
    decode_static_fp4,
    latent_append_fp4,
    sparse_topk_attn_fp4,
    decode_paged_fp4,
    paged_append_fp4,
)

__all__ = [
    "widen",
    "round_to_bf16_bits",
    "kv_append",
    "decode_static",
    "copy_kvcache",
    "trim_kvcache",
    "PagedIndexError",
    "validate_paged",
    "gather_pa_kv_cache",
    "decode_paged",
    "decode_paged_via_gather",
    "sparse_topk_attn",
    "sparse_topk_decode",
    "validate_sparse",
    "e4m3_decode",
    "e4m3_encode",
    "scale_exponent",
    "quantize_rows",
    "kv_append_fp8",
    "decode_static_fp8",
    "decode_paged_fp8",
    "paged_append_fp8",
    "fp4",
    "kv_append_fp4",
    "decode_static_fp4",
    "latent_append_fp8",
    "sparse_topk_attn_fp8",
    "latent_append_fp4",
    "sparse_topk_attn_fp4",
    "decode_paged_fp4",
    "paged_append_fp4",
]
