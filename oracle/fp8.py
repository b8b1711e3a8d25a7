"""FP8 KV cache for decode: E4M3 codes with a power-of-two scale per row (fp64 oracle).

Test infrastructure only.

Source: "FlashMLA on Huawei Ascend", the section on how many VECTOR cores serve one
CUBE core (item 2): at decode time the kernel reads the KV cache in FP8 (or FP4),
dequantises it to bfloat16 and feeds the matrix unit; and the section on the KV
cache layout for decoding: each token's quantised values and its scale belong
together.  The pages fix neither the FP8 variant nor the scale granularity; the
readings taken here are:

* the FP8 format is E4M3 of the OCP 8-bit floating-point specification (sign, 4-bit
  exponent with bias 7, 3-bit mantissa, subnormals, no infinities, S.1111.111 =
  NaN, largest finite value 448);
* one scale per cached row (sequence, head, token) for K and one for V, a power of
  two s = 2^e with e the smallest integer for which max|x| <= 448 * 2^e; a row of
  zeros gets e = 0;
* the code of x is x / s rounded to the nearest E4M3 value, ties to the even code
  (x / s is exact because s is a power of two, and never exceeds 448);
* the cached value is decode(code) * s, which is exactly representable in bf16
  (3 mantissa bits, an exponent shift) unless it falls below bf16's smallest
  subnormal, so attention over the FP8 cache is the attention of the static layout
  over those values;
* the paged pool holds codes ``[num_blocks, block_size, Hkv, D]`` and one scale per
  (block, slot, KV head) ``[num_blocks, block_size, Hkv]`` for K and for V, and the
  new token of sequence b is its last token (position len_b - 1, len_b counting
  it), placed through the block table as every other token;
* the sparse kernel's latent cache (the page's own kernel) holds codes
  ``[B, s_kv, d_qk]`` and one scale per latent row ``[B, s_kv]``: the whole row
  (value and rotary columns alike) shares its scale; a new latent row is quantised
  into position write_pos[b] of its sequence, and the sparse attention runs over
  the dequantised gathered rows.
"""

import math

import numpy as np

from .bf16 import widen
from .paged import _offsets, token_rows, validate_paged
from .sparse import sparse_topk_decode, validate_sparse
from .static_cache import attended_rows, softmax_weighted_sum

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """The value of each E4M3 code (uint8 array) as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


_GRID_CODES = np.arange(0, 0x7F, dtype=np.uint8)          # every finite non-negative code
_GRID = e4m3_decode(_GRID_CODES)                            # increasing, 0 .. 448


def e4m3_encode(x):
    """Nearest E4M3 code of each value in x (|x| <= 448), ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("values beyond 448 have no E4M3 code here")
    a = np.abs(x)
    hi = np.searchsorted(_GRID, a, side="left")             # first grid value >= a
    hi = np.minimum(hi, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_GRID_CODES[hi] % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, _GRID_CODES[hi], _GRID_CODES[lo]).astype(np.uint8)
    code = np.where(a == _GRID[hi], _GRID_CODES[hi], code).astype(np.uint8)
    neg = (np.signbit(x)) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def scale_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    _, ex = math.frexp(amax / E4M3_MAX)                     # amax/448 = f * 2^ex, f in [0.5, 1)
    e = ex
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    return e


def quantize_rows(x_bits):
    """bf16 bit patterns ``[..., D]`` -> (codes uint8 ``[..., D]``, scale float64 ``[...]``)."""
    x = widen(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("a row with NaN or Inf has no E4M3 encoding")
    lead = x.shape[:-1]
    flat = x.reshape(-1, x.shape[-1])
    codes = np.empty(flat.shape, dtype=np.uint8)
    scale = np.empty(flat.shape[0])
    for r in range(flat.shape[0]):
        e = scale_exponent(np.max(np.abs(flat[r])))
        scale[r] = 2.0 ** e
        codes[r] = e4m3_encode(flat[r] / scale[r])
    return codes.reshape(x.shape), scale.reshape(lead)


def dequantize(codes, scale):
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def kv_append_fp8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos, mask=None):
    """Quantise the new token's K and V rows (bf16 bits ``[B, H, D]``) and store the
    codes and scales at row write_pos[b] (codes ``[B, H, cap, D]`` uint8, scales
    ``[B, H, cap]``).  Returns updated copies ``(k_codes, v_codes, k_scale, v_scale,
    mask)``; a position outside ``[0, cap)`` is an error."""
    k_codes, v_codes = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    k_scale, v_scale = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    B, H, cap, D = k_codes.shape
    kq, ks = quantize_rows(k_new)
    vq, vs = quantize_rows(v_new)
    if mask is not None:
        mask = np.array(mask, copy=True)
    for b in range(B):
        pos = int(np.asarray(write_pos).reshape(-1)[b])
        if pos < 0 or pos >= cap:
            raise ValueError(f"write position {pos} outside [0, {cap})")
        k_codes[b, :, pos] = kq[b]
        v_codes[b, :, pos] = vq[b]
        k_scale[b, :, pos] = ks[b]
        v_scale[b, :, pos] = vs[b]
        if mask is not None:
            mask[b, pos] = 1
    return k_codes, v_codes, k_scale, v_scale, mask


def decode_static_fp8(q, k_codes, v_codes, k_scale, v_scale, mask=None, valid_len=None,
                      scale=None):
    """Masked decode attention over the FP8 cache: the attention of the static layout
    over the dequantised rows decode(code) * s (same attended-row rule)."""
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    q = np.asarray(q, dtype=np.float64)
    B, H, cap, D = np.shape(k_codes)
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


def decode_paged_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens,
                     seq_offset=None, scale=None):
    """Paged GQA decode over an FP8 pool: the attention of decode_paged over the
    dequantised rows.  q ``[B, Hq, D]`` (bf16 bits or float); codes uint8
    ``[num_blocks, block_size, Hkv, D]``; scales ``[num_blocks, block_size, Hkv]``.
    Returns ``out [B, Hq, D]`` and ``lse [B, Hq]`` (float64)."""
    q = np.asarray(q)
    qf = widen(q) if q.dtype == np.uint16 else q.astype(np.float64)
    B, Hq, D = qf.shape
    num_blocks, block_size, Hkv, Dk = np.shape(k_codes)
    if Dk != D or np.shape(v_codes) != np.shape(k_codes):
        raise ValueError("codes must be [num_blocks, block_size, Hkv, D]")
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


def paged_append_fp8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_tables, seq_lens,
                     seq_offset=None):
    """Quantise the new token's K and V rows (bf16 bits ``[B, Hkv, D]``) and store them
    as token len_b - 1 of each sequence, at its place in the pool (block table, then
    slot), as kv_append_fp8 does in the static buffer.  Returns updated copies of the
    four arrays; a sequence of length 0 has no place for the token and is an error."""
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



def latent_append_fp8(codes, scale, new_rows, write_pos):
    """Quantise each sequence's new latent row (bf16 bits ``[B, d_qk]``) and store its
    codes and scale at row write_pos[b] of that sequence's cache (codes ``[B, s_kv,
    d_qk]`` uint8, scales ``[B, s_kv]``).  Returns updated copies ``(codes, scale)``; a
    position outside ``[0, s_kv)`` is an error."""
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


def sparse_topk_attn_fp8(q, codes, scale, indices, d_v, sm_scale):
    """Sparse top-k attention over the FP8 latent cache (FlashMLA on Huawei Ascend: the
    decode kernel reads the cache as FP8, dequantises it to bfloat16 and computes as
    before): for each q-token, the rows its indices select are dequantised (code value
    times the row's scale, exact in bf16) and attended exactly as ``sparse_topk_attn``
    attends bf16 rows.

    q       : ``[B, s_q, h_q, d_qk]`` (uint16 bf16 bits, or float)
    codes   : uint8 ``[B, s_kv, d_qk]``;  scale : ``[B, s_kv]``
    indices : ints ``[B, s_q, topk]``
    Returns ``out [B, s_q, h_q, d_v]`` and ``lse [B, s_q, h_q]`` (float64).
    """
    q = np.asarray(q)
    codes = np.asarray(codes)
    scale = np.asarray(scale, dtype=np.float64)
    indices = np.asarray(indices)
    if q.ndim != 4 or indices.ndim != 3 or indices.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [B, s_q, h_q, d_qk] and indices [B, s_q, topk]")
    B, s_q, h_q, _ = q.shape
    if codes.ndim != 3 or codes.shape[0] != B or scale.shape != codes.shape[:2]:
        raise ValueError("codes must be [B, s_kv, d_qk] and scale [B, s_kv]")
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
