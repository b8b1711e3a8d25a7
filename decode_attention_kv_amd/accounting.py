"""Algorithmic byte and flop counts for each operation (what the roofline is priced on).

Only bytes an ideal kernel must move count: valid K/V rows (never the unused
capacity or masked-out rows past the valid length), the query, the output, the
index tensors it reads and the mask entries of attended rows.  Split-K
workspace traffic and re-reads are excluded; they show up as the gap between
these figures and the measured HBM counters.
"""

BF16 = 2
FP32 = 4
INT32 = 4


def kv_layer_bytes(heads, head_dim, rows, elem=BF16):
    """K plus V bytes of ``rows`` cached tokens of one layer (one sequence)."""
    return 2 * heads * rows * head_dim * elem


def copy_kvcache_bytes(layers, heads, seq_len, head_dim, elem=BF16):
    """Bytes of the prefill->generate KV copy: every layer's K and V slice."""
    return layers * kv_layer_bytes(heads, head_dim, seq_len, elem)


def kv_append_bytes(B, H, D, with_mask=True):
    """Read the new K/V rows and write position, write them into the cache (+mask)."""
    new_rows = 2 * B * H * D * BF16
    return 2 * new_rows + B * INT32 + (B * INT32 if with_mask else 0)


def decode_static_bytes(B, H, D, attended, q_elem=FP32, with_mask=True, with_lse=False):
    """One static decode call: ``attended`` is the attended row count per sequence.

    The mask (when given) is read once per attended row of each sequence; it is
    shared by all heads.
    """
    rows = sum(int(x) for x in attended)
    kv = rows * H * D * BF16 * 2
    q = B * H * D * q_elem
    out = B * H * D * FP32 + (B * H * FP32 if with_lse else 0)
    mask = rows * INT32 if with_mask else 0
    valid = B * INT32
    return kv + q + out + mask + valid


def decode_static_fp8_bytes(B, H, D, attended, q_elem=FP32, with_mask=True, with_lse=False):
    """One static decode call over the FP8 cache: one byte per K and V element plus
    one fp32 scale per attended row for K and for V."""
    rows = sum(int(x) for x in attended)
    kv = rows * H * (D * 1 + FP32) * 2
    q = B * H * D * q_elem
    out = B * H * D * FP32 + (B * H * FP32 if with_lse else 0)
    mask = rows * INT32 if with_mask else 0
    return kv + q + out + mask + B * INT32


def kv_append_fp8_bytes(B, H, D, with_mask=True):
    """Read the new bf16 rows and the positions; write codes and scales (+mask)."""
    return 2 * B * H * D * BF16 + B * INT32 + 2 * B * H * (D + FP32) + \
        (B * INT32 if with_mask else 0)


def decode_static_fp4_bytes(B, H, D, attended, q_elem=FP32, with_mask=True, with_lse=False):
    """One static decode call over the FP4 cache: half a byte per K and V element plus
    one fp32 scale per attended row for K and for V."""
    rows = sum(int(x) for x in attended)
    kv = rows * H * (D // 2 + FP32) * 2
    q = B * H * D * q_elem
    out = B * H * D * FP32 + (B * H * FP32 if with_lse else 0)
    mask = rows * INT32 if with_mask else 0
    return kv + q + out + mask + B * INT32


def kv_append_fp4_bytes(B, H, D, with_mask=True):
    """Read the new bf16 rows and the positions; write packed codes and scales (+mask)."""
    return 2 * B * H * D * BF16 + B * INT32 + 2 * B * H * (D // 2 + FP32) + \
        (B * INT32 if with_mask else 0)


def gather_bytes(lengths, Hk, Dk, Hv, Dv, block_size, with_offset=True):
    """gather_pa_kv_cache: read and write every valid token row of K and V."""
    T = sum(int(x) for x in lengths)
    rows = T * (Hk * Dk + Hv * Dv) * BF16
    table = sum(-(-int(x) // block_size) for x in lengths) * INT32
    Q = len(lengths)
    return 2 * rows + table + (Q + 1) * INT32 + (Q * INT32 if with_offset else 0)


def decode_paged_bytes(lengths, Hq, Hkv, D, block_size, q_elem=BF16, with_lse=False):
    """Paged GQA decode: each KV head's valid rows once, q once, out once."""
    T = sum(int(x) for x in lengths)
    B = len(lengths)
    kv = T * Hkv * D * BF16 * 2
    q = B * Hq * D * q_elem
    out = B * Hq * D * FP32 + (B * Hq * FP32 if with_lse else 0)
    table = sum(-(-int(x) // block_size) for x in lengths) * INT32
    return kv + q + out + table + (B + 1) * INT32


def decode_paged_fp8_bytes(lengths, Hq, Hkv, D, block_size, q_elem=BF16, with_lse=False):
    """Paged GQA decode over the FP8 pool: each KV head's valid rows once (D code bytes
    plus a 4-byte scale, for K and for V), q once, out once, table and lengths."""
    T = sum(int(x) for x in lengths)
    B = len(lengths)
    kv = T * Hkv * (D + FP32) * 2
    q = B * Hq * D * q_elem
    out = B * Hq * D * FP32 + (B * Hq * FP32 if with_lse else 0)
    table = sum(-(-int(x) // block_size) for x in lengths) * INT32
    return kv + q + out + table + (B + 1) * INT32


def decode_paged_fp4_bytes(lengths, Hq, Hkv, D, block_size, q_elem=BF16, with_lse=False):
    """Paged GQA decode over the FP4 pool: as decode_paged_fp8_bytes with D / 2 code
    bytes per row."""
    T = sum(int(x) for x in lengths)
    return decode_paged_fp8_bytes(lengths, Hq, Hkv, D, block_size, q_elem, with_lse) - \
        T * Hkv * (D // 2) * 2


def decode_flops(rows, heads_per_row, d_qk, d_v):
    """Multiply-add flops of scores plus the weighted sum (2 per MAC)."""
    return 2 * rows * heads_per_row * (d_qk + d_v)


def sparse_bytes(B, Hq, d_qk, d_v, topk, q_elem=BF16, with_lse=False):
    """Sparse MLA decode: gathered rows once per sequence, q, out, indices."""
    gathered = B * topk * d_qk * BF16
    q = B * Hq * d_qk * q_elem
    out = B * Hq * d_v * FP32 + (B * Hq * FP32 if with_lse else 0)
    return gathered + q + out + B * topk * INT32


def sparse_fp4_bytes(B, Hq, d_qk, d_v, topk, with_lse=False):
    """Sparse MLA decode over the FP4 latent cache: as sparse_fp8_bytes with half a
    byte per value."""
    return sparse_fp8_bytes(B, Hq, d_qk, d_v, topk, with_lse) - B * topk * d_qk // 2


def sparse_fp8_bytes(B, Hq, d_qk, d_v, topk, with_lse=False):
    """Sparse MLA decode over the FP8 latent cache: the gathered rows' codes (one byte
    per value) and row scales once per sequence, q, out, indices."""
    gathered = B * topk * (d_qk + FP32)
    q = B * Hq * d_qk * BF16
    out = B * Hq * d_v * FP32 + (B * Hq * FP32 if with_lse else 0)
    return gathered + q + out + B * topk * INT32


def sparse_macs(B, Hq, d_qk, d_v, topk):
    """Multiply-accumulates of P = Q G^T and O = S G[:, :d_v]."""
    return B * Hq * topk * (d_qk + d_v)


def sparse_flops(B, Hq, d_qk, d_v, topk):
    return 2 * sparse_macs(B, Hq, d_qk, d_v, topk)
