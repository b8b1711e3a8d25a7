"""Paged KV cache: validation, gather_pa_kv_cache and paged GQA decode (fp64 oracle).

Test infrastructure only.

Source: "PyPTO 实现 AscendC GatherPaKvCache（Norm/ND 分支）" (www.mhpn.cn news 2257214):

* section 3.1, tensor contract: ``key_cache [num_blocks, block_size, key_heads,
  key_dim]``, ``value_cache [num_blocks, block_size, value_heads, value_dim]`` (bf16,
  ND), ``block_tables [Q, cols]`` int32, ``seq_lens [Q+1]`` int32 cumulative,
  ``seq_offset [Q]`` int32 or absent; outputs ``key_out [total_tokens, key_heads,
  key_dim]`` and ``value_out [total_tokens, value_heads, value_dim]``.
* section 3.2, gather semantics: for sequence q and token t of it,
  logical block = t // block_size, slot = t % block_size, physical block =
  block_tables[q, table_offset(q) + logical block], and output row
  seq_lens[q] + t receives cache[physical block, slot]; the sequence length is
  seq_lens[q+1] - seq_lens[q]; table_offset(q) = seq_offset[q] // block_size, or 0
  when no offset is given.  (The extraction dropped the '+' signs; the reading
  above is the only one that types.)
* section 3.3, shape constraints: cumulative seq_lens of length Q+1 starting at 0
  and non-decreasing, seq_offset non-negative and divisible by block_size, every
  block-table entry that is used lies in [0, num_blocks).
* section 7: only the cumulative form of seq_lens is accepted; any other is an
  error.

Paged decode attention applies the masked-softmax definition of the static
oracle to the rows the table walk yields (valid length = the sequence length, no
mask); query head h reads KV head ``h // (Hq / Hkv)`` -- several query heads share
one KV head (the NPU article's closing part on GQA: "several Q heads share the
same KV tile"); contiguous groups are the reading taken.
"""

import numpy as np

from .bf16 import widen
from .static_cache import softmax_weighted_sum


class PagedIndexError(ValueError):
    """An index tensor (seq_lens, seq_offset, block_tables) breaks the contract."""


def _offsets(seq_offset, Q):
    if seq_offset is None:
        return np.zeros(Q, dtype=np.int64)
    return np.asarray(seq_offset, dtype=np.int64).reshape(-1)


def validate_paged(block_tables, seq_lens, seq_offset, num_blocks, block_size):
    """Raise PagedIndexError unless the index tensors satisfy section 3.3."""
    block_tables = np.asarray(block_tables)
    if block_tables.ndim != 2:
        raise PagedIndexError("block_tables must be [Q, cols]")
    Q, cols = block_tables.shape
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    if seq_lens.shape != (Q + 1,):
        raise PagedIndexError("only cumulative seq_lens of length Q + 1 is supported")
    if seq_lens[0] != 0:
        raise PagedIndexError("cumulative seq_lens must start at 0")
    if np.any(np.diff(seq_lens) < 0):
        raise PagedIndexError("cumulative seq_lens must be non-decreasing")
    offsets = _offsets(seq_offset, Q)
    if offsets.shape != (Q,):
        raise PagedIndexError("seq_offset must be [Q]")
    if np.any(offsets < 0) or np.any(offsets % block_size != 0):
        raise PagedIndexError("seq_offset must be non-negative multiples of block_size")
    for q in range(Q):
        length = int(seq_lens[q + 1] - seq_lens[q])
        first = int(offsets[q] // block_size)
        used = -(-length // block_size)
        if used == 0:
            continue
        if first + used > cols:
            raise PagedIndexError(f"sequence {q} needs table columns beyond {cols}")
        ids = block_tables[q, first:first + used]
        if np.any(ids < 0) or np.any(ids >= num_blocks):
            raise PagedIndexError(f"sequence {q} uses a block id outside [0, {num_blocks})")


def token_rows(q, block_tables, seq_lens, offsets, block_size):
    """(physical block, slot) of every token of sequence q, in token order."""
    length = int(seq_lens[q + 1] - seq_lens[q])
    first = int(offsets[q] // block_size)
    t = np.arange(length)
    logical = t // block_size
    slot = t % block_size
    phys = np.asarray(block_tables)[q, first + logical]
    return phys, slot


def gather_pa_kv_cache(key_cache, value_cache, block_tables, seq_lens, seq_offset=None):
    """Collect each sequence's paged rows into contiguous outputs (bit copy).

    key_cache   : uint16 bf16 bits ``[num_blocks, block_size, Hk, Dk]``
    value_cache : uint16 bf16 bits ``[num_blocks, block_size, Hv, Dv]``
    Returns ``key_out [T, Hk, Dk]`` and ``value_out [T, Hv, Dv]`` (uint16), where
    ``T = seq_lens[Q]``.
    """
    key_cache = np.asarray(key_cache)
    value_cache = np.asarray(value_cache)
    num_blocks, block_size = key_cache.shape[:2]
    if value_cache.shape[:2] != (num_blocks, block_size):
        raise PagedIndexError("key_cache and value_cache must agree on num_blocks, block_size")
    validate_paged(block_tables, seq_lens, seq_offset, num_blocks, block_size)
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    Q = seq_lens.shape[0] - 1
    offsets = _offsets(seq_offset, Q)
    total = int(seq_lens[Q])
    key_out = np.zeros((total,) + key_cache.shape[2:], dtype=key_cache.dtype)
    value_out = np.zeros((total,) + value_cache.shape[2:], dtype=value_cache.dtype)
    for q in range(Q):
        base = int(seq_lens[q])
        phys, slot = token_rows(q, block_tables, seq_lens, offsets, block_size)
        for t in range(phys.shape[0]):
            key_out[base + t] = key_cache[phys[t], slot[t]]
            value_out[base + t] = value_cache[phys[t], slot[t]]
    return key_out, value_out


def _as_f64(x):
    x = np.asarray(x)
    return widen(x) if x.dtype == np.uint16 else x.astype(np.float64)


def decode_paged(q, key_cache, value_cache, block_tables, seq_lens, seq_offset=None,
                 scale=None):
    """Paged GQA decode attention, walking the block table directly.

    q           : ``[B, Hq, D]`` (uint16 bf16 bits, or float)
    key_cache   : uint16 bf16 bits ``[num_blocks, block_size, Hkv, D]``
    value_cache : same shape as key_cache
    seq_lens    : cumulative ``[B + 1]``; sequence b has seq_lens[b+1]-seq_lens[b] rows
    Returns ``out [B, Hq, D]`` and ``lse [B, Hq]`` (float64).
    """
    qf = _as_f64(q)
    B, Hq, D = qf.shape
    num_blocks, block_size, Hkv, Dk = np.shape(key_cache)
    if Dk != D or np.shape(value_cache) != np.shape(key_cache):
        raise ValueError("key/value cache must be [num_blocks, block_size, Hkv, D]")
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
        K = widen(np.asarray(key_cache)[phys, slot])      # [len, Hkv, D]
        V = widen(np.asarray(value_cache)[phys, slot])
        for h in range(Hq):
            g = h // group
            s = scale * (K[:, g, :] @ qf[b, h])
            out[b, h], lse[b, h] = softmax_weighted_sum(s, V[:, g, :])
    return out, lse


def decode_paged_via_gather(q, key_cache, value_cache, block_tables, seq_lens,
                            seq_offset=None, scale=None):
    """Second, independent route to paged decode: gather, then dense attention.

    Used only to cross-check ``decode_paged`` (two oracle paths must agree).
    """
    qf = _as_f64(q)
    B, Hq, D = qf.shape
    Hkv = np.shape(key_cache)[2]
    group = Hq // Hkv
    key_out, value_out = gather_pa_kv_cache(key_cache, value_cache, block_tables,
                                            seq_lens, seq_offset)
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        lo, hi = int(seq_lens[b]), int(seq_lens[b + 1])
        K = widen(key_out[lo:hi])
        V = widen(value_out[lo:hi])
        for g in range(Hkv):
            for j in range(group):
                h = g * group + j
                s = scale * (K[:, g, :] @ qf[b, h])
                out[b, h], lse[b, h] = softmax_weighted_sum(s, V[:, g, :])
    return out, lse
