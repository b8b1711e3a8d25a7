"""FP4 KV cache for decode: E2M1 codes with a power-of-two scale per row (fp64 oracle).

Test infrastructure only.

Source: "FlashMLA on Huawei Ascend", the section on how many VECTOR cores serve one
CUBE core (item 2): at decode time the kernel reads the KV cache in FP8 or FP4 and
dequantises it to bfloat16.  The page fixes neither the FP4 variant nor the scale;
the readings taken here follow the FP8 cache's (one power-of-two scale per cached
row, for K and for V, kept in its own array):

* the FP4 format is E2M1 of the OCP microscaling specification: sign, 2-bit exponent
  with bias 1, 1-bit mantissa, one subnormal (0.5), no infinities or NaN; the
  magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* the scale of a row is s = 2^e with e the smallest integer for which
  max|x| <= 6 * 2^e (a row of zeros gets e = 0); the code of x is x / s (exact)
  rounded to the nearest E2M1 value, ties to the even code, zero results as +0;
* two codes share a byte, element 2i in the low four bits and 2i + 1 in the high
  four bits (the microscaling specification's packing);
* the cached value is decode(code) * s, exactly representable in bf16, so the
  attention over the FP4 cache is the attention of the static layout over those
  values;
* the paged pool in FP4 holds packed codes ``[num_blocks, block_size, Hkv, D/2]`` and
  one scale per (block, slot, KV head) for K and for V, with the new token of a
  sequence placed as in the FP8 pool (its last position, through the table);
* the sparse kernel's latent cache in FP4 holds packed codes ``[B, s_kv, d_qk/2]``
  and one scale per latent row ``[B, s_kv]`` for all its columns, as the FP8
  latent cache does; the sparse attention runs over the dequantised gathered rows.
"""

import math

import numpy as np

from .bf16 import widen
from .paged import _offsets, token_rows, validate_paged
from .sparse import sparse_topk_decode, validate_sparse
from .static_cache import attended_rows, softmax_weighted_sum

E2M1_MAX = 6.0
_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(nibbles):
    """4-bit codes (any integer array, values 0..15) -> float64 values."""
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    mag = _MAGS[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x):
    """Values with |x| <= 6 -> the nearest E2M1 code (ties to the even code; a
    result of zero is the +0 code)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E2M1_MAX):
        raise ValueError("E2M1 input outside [-6, 6]")
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 0, 7)   # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _MAGS[hi], hi, code).astype(np.uint8)
    neg = np.signbit(x) & (code != 0)
    return np.where(neg, code | 8, code).astype(np.uint8)


def scale_exponent(amax):
    """Smallest integer e with amax <= 6 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    _, e = math.frexp(amax / E2M1_MAX)
    while amax <= E2M1_MAX * 2.0 ** (e - 1):
        e -= 1
    while amax > E2M1_MAX * 2.0 ** e:
        e += 1
    return e


def pack(codes):
    """4-bit codes ``[..., D]`` (D even) -> bytes ``[..., D/2]``, element 2i low."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """Bytes ``[..., D/2]`` -> 4-bit codes ``[..., D]``."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_rows(x_bits):
    """bf16 bit patterns ``[..., D]`` -> (packed codes uint8 ``[..., D/2]``, scale
    float64 ``[...]``)."""
    x = widen(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("a row with NaN or Inf has no E2M1 encoding")
    if x.shape[-1] % 2:
        raise ValueError("the row length must be even")
    lead = x.shape[:-1]
    flat = x.reshape(-1, x.shape[-1])
    codes = np.empty(flat.shape, dtype=np.uint8)
    scale = np.empty(flat.shape[0])
    for r in range(flat.shape[0]):
        e = scale_exponent(np.max(np.abs(flat[r])))
        scale[r] = 2.0 ** e
        codes[r] = e2m1_encode(flat[r] / scale[r])
    return pack(codes.reshape(x.shape)), scale.reshape(lead)


def dequantize(packed, scale):
    return e2m1_decode(unpack(packed)) * np.asarray(scale, dtype=np.float64)[..., None]


def kv_append_fp4(k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos, mask=None):
    """Quantise the new token's K and V rows (bf16 bits ``[B, H, D]``) and store the
    packed codes and scales at row write_pos[b] (codes ``[B, H, cap, D/2]`` uint8,
    scales ``[B, H, cap]``).  Returns updated copies ``(k_codes, v_codes, k_scale,
    v_scale, mask)``; a position outside ``[0, cap)`` is an error."""
    k_codes, v_codes = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    k_scale, v_scale = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    B, H, cap, _ = k_codes.shape
    kq, ks = quantize_rows(k_new)
    vq, vs = quantize_rows(v_new)
    if mask is not None:
        mask = np.array(mask, copy=True)
    for b in range(B):
        pos = int(np.asarray(write_pos).reshape(-1)[b])
        if pos < 0 or pos >= cap:
            raise ValueError(f"write position {pos} outside [0, {cap})")
        k_codes[b, :, pos], v_codes[b, :, pos] = kq[b], vq[b]
        k_scale[b, :, pos], v_scale[b, :, pos] = ks[b], vs[b]
        if mask is not None:
            mask[b, pos] = 1
    return k_codes, v_codes, k_scale, v_scale, mask


def decode_static_fp4(q, k_codes, v_codes, k_scale, v_scale, mask=None, valid_len=None,
                      scale=None):
    """Masked decode attention over the FP4 cache: the attention of the static layout
    over the dequantised rows decode(code) * s (same attended-row rule)."""
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    q = np.asarray(q, dtype=np.float64)
    B, H, cap, half = np.shape(k_codes)
    D = 2 * half
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        rows = attended_rows(cap, None if mask is None else mask[b],
                             None if valid_len is None else valid_len[b])
        for h in range(H):
            K = dequantize(k_codes[b, h, rows], k_scale[b, h, rows])
            V = dequantize(v_codes[b, h, rows], v_scale[b, h, rows])
            out[b, h], lse[b, h] = softmax_weighted_sum(scale * (K @ q[b, h]), V)
    return out, lse


def latent_append_fp4(codes, scale, new_rows, write_pos):
    """Quantise each sequence's new latent row (bf16 bits ``[B, d_qk]``) and store its
    packed codes and scale at row write_pos[b] of that sequence's cache (codes
    ``[B, s_kv, d_qk/2]`` uint8, scales ``[B, s_kv]``).  Returns updated copies
    ``(codes, scale)``; a position outside ``[0, s_kv)`` is an error."""
    codes, scale = np.array(codes, copy=True), np.array(scale, copy=True)
    B, s_kv, _ = codes.shape
    rq, rs = quantize_rows(new_rows)
    for b in range(B):
        pos = int(np.asarray(write_pos).reshape(-1)[b])
        if pos < 0 or pos >= s_kv:
            raise ValueError(f"write position {pos} outside [0, {s_kv})")
        codes[b, pos] = rq[b]
        scale[b, pos] = rs[b]
    return codes, scale


def sparse_topk_attn_fp4(q, codes, scale, indices, d_v, sm_scale):
    """Sparse top-k attention over the FP4 latent cache (FlashMLA on Huawei Ascend: the
    decode kernel reads the cache as FP8 or FP4 and dequantises it to bfloat16): for
    each q-token, the rows its indices select are dequantised (code value times the
    row's scale, exact in bf16) and attended exactly as ``sparse_topk_attn`` attends
    bf16 rows.

    q       : ``[B, s_q, h_q, d_qk]`` (uint16 bf16 bits, or float)
    codes   : uint8 ``[B, s_kv, d_qk/2]`` (element 2i in the low four bits);
    scale   : ``[B, s_kv]``;  indices : ints ``[B, s_q, topk]``
    Returns ``out [B, s_q, h_q, d_v]`` and ``lse [B, s_q, h_q]`` (float64).
    """
    q = np.asarray(q)
    codes = np.asarray(codes)
    scale = np.asarray(scale, dtype=np.float64)
    indices = np.asarray(indices)
    if q.ndim != 4 or indices.ndim != 3 or indices.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [B, s_q, h_q, d_qk] and indices [B, s_q, topk]")
    B, s_q, h_q, d_qk = q.shape
    if (codes.ndim != 3 or codes.shape[0] != B or 2 * codes.shape[2] != d_qk
            or scale.shape != codes.shape[:2]):
        raise ValueError("codes must be [B, s_kv, d_qk/2] and scale [B, s_kv]")
    validate_sparse(indices, codes.shape[1])
    topk = indices.shape[2]
    out = np.zeros((B, s_q, h_q, d_v))
    lse = np.full((B, s_q, h_q), -np.inf)
    for b in range(B):
        for t in range(s_q):
            idx = indices[b, t]
            rows = dequantize(codes[b][idx], scale[b][idx])        # [topk, d_qk]
            o, l = sparse_topk_decode(q[b, t][None], rows[None], np.arange(topk)[None],
                                      d_v, sm_scale)
            out[b, t], lse[b, t] = o[0], l[0]
    return out, lse


def decode_paged_fp4(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens,
                     seq_offset=None, scale=None):
    """Paged GQA decode over an FP4 pool: the attention of decode_paged over the
    dequantised rows.  q ``[B, Hq, D]`` (bf16 bits or float); packed codes uint8
    ``[num_blocks, block_size, Hkv, D/2]``; scales ``[num_blocks, block_size, Hkv]``.
    Returns ``out [B, Hq, D]`` and ``lse [B, Hq]`` (float64)."""
    q = np.asarray(q)
    qf = widen(q) if q.dtype == np.uint16 else q.astype(np.float64)
    B, Hq, D = qf.shape
    num_blocks, block_size, Hkv, half = np.shape(k_codes)
    if 2 * half != D or np.shape(v_codes) != np.shape(k_codes):
        raise ValueError("codes must be [num_blocks, block_size, Hkv, D/2]")
    if np.shape(k_scale) != (num_blocks, block_size, Hkv) or np.shape(v_scale) != np.shape(k_scale):
        raise ValueError("scales must be [num_blocks, block_size, Hkv]")
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    validate_paged(block_tables, seq_lens, seq_offset, num_blocks, block_size)
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    offsets = _offsets(seq_offset, B)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        phys, slot = token_rows(b, block_tables, seq_lens, offsets, block_size)
        K = dequantize(np.asarray(k_codes)[phys, slot], np.asarray(k_scale)[phys, slot])
        V = dequantize(np.asarray(v_codes)[phys, slot], np.asarray(v_scale)[phys, slot])
        for h in range(Hq):
            g = h // group
            out[b, h], lse[b, h] = softmax_weighted_sum(scale * (K[:, g, :] @ qf[b, h]),
                                                        V[:, g, :])
    return out, lse


def paged_append_fp4(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_tables, seq_lens,
                     seq_offset=None):
    """Quantise the new token's K and V rows (bf16 bits ``[B, Hkv, D]``) to E2M1 and
    store them as token len_b - 1 of each sequence, at its place in the pool (block
    table, then slot).  Returns updated copies of the four arrays; a sequence of
    length 0 has no place for the token and is an error."""
    k_codes, v_codes = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    k_scale, v_scale = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    num_blocks, block_size = k_codes.shape[:2]
    validate_paged(block_tables, seq_lens, seq_offset, num_blocks, block_size)
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    B = seq_lens.shape[0] - 1
    offsets = _offsets(seq_offset, B)
    kq, ks = quantize_rows(k_new)
    vq, vs = quantize_rows(v_new)
    for b in range(B):
        phys, slot = token_rows(b, block_tables, seq_lens, offsets, block_size)
        if phys.shape[0] == 0:
            raise ValueError(f"sequence {b} has length 0: no place for its new token")
        p, sl = phys[-1], slot[-1]
        k_codes[p, sl], v_codes[p, sl] = kq[b], vq[b]
        k_scale[p, sl], v_scale[p, sl] = ks[b], vs[b]
    return k_codes, v_codes, k_scale, v_scale
