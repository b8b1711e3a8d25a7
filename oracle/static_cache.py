"""Static preallocated KV buffer: append and masked decode attention (fp64 oracle).

Test infrastructure only.

Sources (all on the OpenVINO community article on running LLMs on the Intel NPU,
openvinohackathon.51openlab.com article 882, and its retelling "NPU 上的 LLM 推理：
KV Cache 与软件栈", jonathanding.github.io):

* Part 1, "Solution: preallocation + attention mask": the cache is one fixed
  buffer ``[batch, heads, capacity, head_dim]`` with capacity
  MAX_PROMPT_LEN + MIN_RESPONSE_LEN = 1024 + 128 = 1152; a 0/1 mask as long as the
  sequence axis marks valid rows; softmax sees -inf where mask = 0, so those rows
  get weight zero and their contents (zero or garbage) are ignored.
* Part 2, the generate loop (``update_kvcache_for``): each step writes only the
  new token's K and V into the next free row and bumps the stored-row counter.
* "Attention on the NPU" -> decomposed SDPA: Q x K^T, times the scale, plus the
  mask, softmax, times V; "incremental SDPA": the decode case with one query row.
* The cuTile tile example divides scores by sqrt(HEAD_DIM), fixing the default
  scale 1/sqrt(d).

Reading taken where the pages leave a step open: a row t of sequence b is
attended iff ``t < valid_len[b]`` and ``mask[b, t] != 0`` (either input may be
absent, not both); rows outside that set are excluded from the sum, never
multiplied by zero, so NaN or Inf stored there cannot reach the output.  A
sequence with no attended row returns zeros and lse = -inf.
"""

import numpy as np

from .bf16 import widen


def kv_append(k_cache, v_cache, k_new, v_new, write_pos, mask=None):
    """Write one new K/V row per sequence at its write position.

    k_cache, v_cache : uint16 bf16 bits ``[B, H, cap, D]``
    k_new, v_new     : uint16 bf16 bits ``[B, H, D]`` (the new token, every head)
    write_pos        : ints ``[B]``, the row to write (the number of rows stored
                       so far); must lie in ``[0, cap)``
    mask             : int ``[B, cap]`` or None; when given, ``mask[b, pos] = 1``

    Returns updated copies ``(k_cache, v_cache, mask)``; inputs are not modified.
    A position outside the buffer is an error (the page: a conversation longer than
    the capacity either errors or is truncated and re-prefilled).
    """
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    B, H, cap, D = k_cache.shape
    if v_cache.shape != (B, H, cap, D):
        raise ValueError("k_cache and v_cache shapes differ")
    if np.shape(k_new) != (B, H, D) or np.shape(v_new) != (B, H, D):
        raise ValueError("new rows must be [B, H, D]")
    write_pos = np.asarray(write_pos).reshape(-1)
    if write_pos.shape != (B,):
        raise ValueError("write_pos must be [B]")
    if mask is not None:
        mask = np.array(mask, copy=True)
        if mask.shape != (B, cap):
            raise ValueError("mask must be [B, cap]")
    for b in range(B):
        pos = int(write_pos[b])
        if pos < 0 or pos >= cap:
            raise ValueError(f"write position {pos} outside [0, {cap})")
        k_cache[b, :, pos, :] = k_new[b]
        v_cache[b, :, pos, :] = v_new[b]
        if mask is not None:
            mask[b, pos] = 1
    return k_cache, v_cache, mask


def attended_rows(cap, mask_row, valid_len):
    """Indices of the rows one sequence attends (ascending)."""
    limit = cap if valid_len is None else int(valid_len)
    if limit < 0 or limit > cap:
        raise ValueError(f"valid length {limit} outside [0, {cap}]")
    rows = np.arange(limit)
    if mask_row is not None:
        rows = rows[np.asarray(mask_row)[:limit] != 0]
    return rows


def softmax_weighted_sum(scores, values):
    """Two-pass softmax of ``scores [n]`` applied to ``values [n, d]``.

    Returns ``(out [d], lse)`` with ``lse = log(sum(exp(scores)))`` (natural log).
    Subtracting the maximum is only for range; the result is the plain softmax.
    """
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf
    m = np.max(scores)
    w = np.exp(scores - m)
    total = np.sum(w)
    return (w @ values) / total, m + np.log(total)


def decode_static(q, k_cache, v_cache, mask=None, valid_len=None, scale=None):
    """Decode attention of one new query row per (sequence, head).

    q        : float ``[B, H, D]`` (the page's fp32 query)
    k_cache  : uint16 bf16 bits ``[B, H, cap, D]``
    v_cache  : uint16 bf16 bits ``[B, H, cap, D]``
    mask     : int ``[B, cap]`` 0/1 (nonzero counts as 1), or None
    valid_len: int ``[B]``, or None; at least one of mask / valid_len is given
    scale    : float, default ``1 / sqrt(D)``

    Returns ``out`` float64 ``[B, H, D]`` and ``lse`` float64 ``[B, H]`` where for the
    attended rows T: ``s_t = scale * q . K_t``, ``out = sum_t softmax(s)_t V_t`` and
    ``lse = log sum_t exp(s_t)``.
    """
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    q = np.asarray(q, dtype=np.float64)
    B, H, cap, D = np.shape(k_cache)
    if q.shape != (B, H, D):
        raise ValueError("q must be [B, H, D]")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        rows = attended_rows(
            cap,
            None if mask is None else mask[b],
            None if valid_len is None else valid_len[b],
        )
        for h in range(H):
            K = widen(k_cache[b, h, rows, :])
            V = widen(v_cache[b, h, rows, :])
            s = scale * (K @ q[b, h])
            out[b, h], lse[b, h] = softmax_weighted_sum(s, V)
    return out, lse


def copy_kvcache(src, dst, lengths, mask=None):
    """Prefill -> generate hand-over of the KV cache.

    The prefill model's present K/V tensors have capacity S_src (the page: 1024),
    the generate model's past tensors capacity S_dst (1152); for every layer's K and
    V, the valid rows [0, len_b) of sequence b are copied from present to past at the
    same rows (Part 2, step 3 of the generate flow: a slice per tensor, 32 layers x 2
    tensors copied in parallel; "Current limitations": the copy is 512 MB at 7B with
    1024 rows).  Rows of past at and after len_b keep their contents.

    src, dst : lists of equal length; src[i] uint16 bits ``[B, H, S_src, D]``,
               dst[i] uint16 bits ``[B, H, S_dst, D]``
    lengths  : ints ``[B]`` in ``[0, min(S_src, S_dst)]``
    mask     : int ``[B, S_dst]`` or None; when given it becomes 1 for the copied
               rows and 0 for the rest (the stored-row count is len_b)

    Returns ``(new dst list, new mask)``; inputs are not modified.
    """
    if len(src) != len(dst):
        raise ValueError("src and dst must list the same number of tensors")
    lengths = np.asarray(lengths).reshape(-1)
    out = []
    for s, d in zip(src, dst):
        s = np.asarray(s)
        d = np.array(d, copy=True)
        B, H, S_src, D = s.shape
        if d.shape[:2] != (B, H) or d.shape[3] != D:
            raise ValueError("src and dst differ in batch, heads or head_dim")
        S_dst = d.shape[2]
        if lengths.shape != (B,):
            raise ValueError("lengths must be [B]")
        for b in range(B):
            n = int(lengths[b])
            if n < 0 or n > min(S_src, S_dst):
                raise ValueError(f"length {n} outside [0, {min(S_src, S_dst)}]")
            d[b, :, :n, :] = s[b, :, :n, :]
        out.append(d)
    if mask is not None:
        mask = np.array(mask, copy=True)
        if mask.shape[0] != lengths.shape[0]:
            raise ValueError("mask must be [B, S_dst]")
        for b in range(mask.shape[0]):
            mask[b, :] = 0
            mask[b, :int(lengths[b])] = 1
    return out, mask


def trim_kvcache(mask, new_len):
    """Roll the stored rows of each sequence back to ``new_len[b]``.

    The page's speculative-decoding support cuts the cache back to the last accepted
    position (``trim_kvcache_for_speculative_decoding``, NPUW deployment features);
    with the 0/1 mask that means rows at and after new_len[b] stop counting.  Earlier
    entries are unchanged and the row contents are left as they are (the mask hides
    them).  new_len[b] must lie in [0, S].
    """
    mask = np.array(mask, copy=True)
    new_len = np.asarray(new_len).reshape(-1)
    if new_len.shape != (mask.shape[0],):
        raise ValueError("new_len must be [B]")
    for b in range(mask.shape[0]):
        n = int(new_len[b])
        if n < 0 or n > mask.shape[1]:
            raise ValueError(f"length {n} outside [0, {mask.shape[1]}]")
        mask[b, n:] = 0
    return mask
