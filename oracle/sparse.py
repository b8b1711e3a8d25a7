"""Top-k sparse MLA-style decode attention (fp64 oracle).

Test infrastructure only.

Source: "FlashMLA на Huawei Ascend: ядро разреженного внимания изнутри"
(ai.flicky.cc, translation of DeepSeek's FlashMLA note), section "Mathematical
formulation": each q-token is independent; given ``Q [h_q, d_qk]``,
``KV [s_kv, d_qk]``, ``indices [topk]`` and a scalar ``sm_scale``:

    gathered = KV.index_select(indices)            [topk, d_qk]
    P        = Q @ gathered^T                      [h_q, topk]
    S        = softmax(P * sm_scale, dim=-1)       [h_q, topk]
    out      = S @ gathered[:, :d_v]               [h_q, d_v]

All heads of one q-token share the gathered rows (the latent KV); the value is
the first d_v columns of the same rows.  index_select repeats duplicated indices
(a row chosen twice counts twice) and an index outside [0, s_kv) is an error.
Readings taken: one latent cache per sequence, ``KV [B, s_kv, d_qk]`` with
``indices [B, topk]``; the log-sum-exp returned is of the scaled scores.
"""

import numpy as np

from .bf16 import widen
from .static_cache import softmax_weighted_sum


def validate_sparse(indices, s_kv):
    """Raise ValueError if any index lies outside [0, s_kv)."""
    idx = np.asarray(indices)
    if np.any(idx < 0) or np.any(idx >= s_kv):
        raise ValueError(f"sparse index outside [0, {s_kv})")


def _as_f64(x):
    x = np.asarray(x)
    return widen(x) if x.dtype == np.uint16 else x.astype(np.float64)


def sparse_topk_decode(q, kv, indices, d_v, sm_scale):
    """Sparse decode for every sequence b.

    q       : ``[B, h_q, d_qk]`` (uint16 bf16 bits, or float)
    kv      : uint16 bf16 bits ``[B, s_kv, d_qk]``
    indices : ints ``[B, topk]``
    Returns ``out [B, h_q, d_v]`` and ``lse [B, h_q]`` (float64).
    """
    qf = _as_f64(q)
    B, h_q, d_qk = qf.shape
    kv = np.asarray(kv)
    if kv.shape[0] != B or kv.shape[2] != d_qk:
        raise ValueError("kv must be [B, s_kv, d_qk]")
    if not 0 < d_v <= d_qk:
        raise ValueError("d_v must lie in (0, d_qk]")
    s_kv = kv.shape[1]
    indices = np.asarray(indices)
    validate_sparse(indices, s_kv)
    out = np.zeros((B, h_q, d_v))
    lse = np.full((B, h_q), -np.inf)
    for b in range(B):
        gathered = _as_f64(kv[b][indices[b]])     # [topk, d_qk], duplicates repeat
        P = qf[b] @ gathered.T                    # [h_q, topk]
        values = gathered[:, :d_v]
        for h in range(h_q):
            out[b, h], lse[b, h] = softmax_weighted_sum(P[h] * sm_scale, values)
    return out, lse


def sparse_topk_attn(q, kv, indices, d_v, sm_scale):
    """The page's kernel in general form (FlashMLA on Huawei Ascend, "Reminder of the
    algorithm" and "Mathematical formulation"): a sequence has several q-tokens, each
    with its own index list into the sequence's one latent cache, and the q-tokens are
    computed separately -- each one is exactly ``sparse_topk_decode`` of that token.

    q       : ``[B, s_q, h_q, d_qk]`` (uint16 bf16 bits, or float)
    kv      : uint16 bf16 bits ``[B, s_kv, d_qk]``
    indices : ints ``[B, s_q, topk]``
    Returns ``out [B, s_q, h_q, d_v]`` and ``lse [B, s_q, h_q]`` (float64).
    """
    q = np.asarray(q)
    indices = np.asarray(indices)
    if q.ndim != 4 or indices.ndim != 3 or indices.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [B, s_q, h_q, d_qk] and indices [B, s_q, topk]")
    B, s_q, h_q, _ = q.shape
    out = np.zeros((B, s_q, h_q, d_v))
    lse = np.full((B, s_q, h_q), -np.inf)
    for t in range(s_q):
        out[:, t], lse[:, t] = sparse_topk_decode(q[:, t], kv, indices[:, t], d_v, sm_scale)
    return out, lse

