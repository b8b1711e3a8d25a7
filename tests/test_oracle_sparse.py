"""Pins of the sparse top-k MLA-style decode oracle -- CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import round_to_bf16_bits, widen


def random_bits(rng, shape):
    return round_to_bf16_bits(rng.standard_normal(shape))


def test_full_index_reduces_to_dense_attention_library_routine():
    """topk = s_kv with indices 0..s_kv-1: every head is plain attention of its
    query over K = KV, V = KV[:, :d_v]; checked against torch SDPA in float64."""
    rng = np.random.default_rng(30)
    B, Hq, s_kv, d_qk, d_v = 2, 5, 37, 24, 16
    kv = random_bits(rng, (B, s_kv, d_qk))
    q = random_bits(rng, (B, Hq, d_qk))
    idx = np.tile(np.arange(s_kv, dtype=np.int32), (B, 1))
    scale = 0.21
    out, lse = oracle.sparse_topk_decode(q, kv, idx, d_v, scale)
    for b in range(B):
        K = torch.from_numpy(widen(kv[b])).view(1, 1, s_kv, d_qk)
        V = torch.from_numpy(widen(kv[b])[:, :d_v].copy()).view(1, 1, s_kv, d_v)
        Q = torch.from_numpy(widen(q[b])).view(1, 1, Hq, d_qk)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        assert np.max(np.abs(out[b] - ref.view(Hq, d_v).numpy())) < 1e-12
        s = scale * (widen(q[b]) @ widen(kv[b]).T)
        assert np.allclose(lse[b], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-12)


def test_index_order_does_not_matter():
    rng = np.random.default_rng(31)
    B, Hq, s_kv, d_qk, d_v, topk = 2, 3, 100, 16, 8, 20
    kv = random_bits(rng, (B, s_kv, d_qk))
    q = random_bits(rng, (B, Hq, d_qk))
    idx = np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(B)])
    a = oracle.sparse_topk_decode(q, kv, idx, d_v, 0.25)
    b = oracle.sparse_topk_decode(q, kv, idx[:, ::-1].copy(), d_v, 0.25)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-14)
    assert np.allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_duplicated_index_counts_twice():
    """index_select repeats rows: a duplicate equals adding ln 2 to that row's score."""
    rng = np.random.default_rng(32)
    Hq, s_kv, d_qk, d_v = 4, 12, 8, 4
    kv = random_bits(rng, (1, s_kv, d_qk))
    q = random_bits(rng, (1, Hq, d_qk))
    idx = np.array([[3, 7, 7, 10]])
    out, lse = oracle.sparse_topk_decode(q, kv, idx, d_v, 0.5)
    G = widen(kv[0, [3, 7, 10]])
    s = 0.5 * (widen(q[0]) @ G.T)
    s[:, 1] += math.log(2.0)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (w @ G[:, :d_v]) / w.sum(axis=1, keepdims=True)
    assert np.allclose(out[0], ref, rtol=0, atol=1e-14)
    assert np.allclose(lse[0], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-13)


def test_single_index_returns_that_value_row():
    rng = np.random.default_rng(33)
    kv = random_bits(rng, (1, 9, 12))
    q = random_bits(rng, (1, 3, 12))
    out, lse = oracle.sparse_topk_decode(q, kv, np.array([[6]]), 5, 0.1)
    assert np.array_equal(out[0], np.broadcast_to(widen(kv[0, 6, :5]), (3, 5)))
    assert np.allclose(lse[0], 0.1 * (widen(q[0]) @ widen(kv[0, 6])), rtol=0, atol=1e-15)


def test_value_is_the_leading_columns_of_the_gathered_rows():
    """Zero query -> uniform weights -> out = mean of gathered rows' first d_v columns."""
    rng = np.random.default_rng(34)
    kv = random_bits(rng, (1, 50, 10))
    idx = np.array([[4, 9, 33, 2, 41]])
    out, lse = oracle.sparse_topk_decode(np.zeros((1, 2, 10)), kv, idx, 6, 1.0)
    assert np.allclose(out[0], widen(kv[0, idx[0], :6]).mean(axis=0), rtol=0, atol=1e-15)
    assert np.allclose(lse, math.log(5), atol=1e-15)


@pytest.mark.parametrize("bad", [-1, 50])
def test_out_of_range_index_is_an_error(bad):
    kv = np.zeros((1, 50, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.sparse_topk_decode(np.zeros((1, 1, 4)), kv, np.array([[0, bad]]), 2, 1.0)


# ------------------------------------------------------- several q-tokens per sequence


def test_tokens_attend_through_their_own_indices_brute_force():
    """Two q-tokens of one sequence, each with its own index list over the one latent
    cache: every (token, head) output is the softmax-weighted mean written out with
    math.exp over that token's gathered rows (no array library in the check)."""
    rng = np.random.default_rng(71)
    B, s_q, h_q, d_qk, d_v, s_kv = 2, 2, 2, 6, 4, 9
    kv = random_bits(rng, (B, s_kv, d_qk))
    q = random_bits(rng, (B, s_q, h_q, d_qk))
    idx = np.stack([np.stack([rng.choice(s_kv, 4, replace=False) for _ in range(s_q)])
                    for _ in range(B)])
    out, lse = oracle.sparse_topk_attn(q, kv, idx, d_v, 0.5)
    kvf, qf = widen(kv), widen(q)
    for b in range(B):
        for t in range(s_q):
            for h in range(h_q):
                rows = [kvf[b, i] for i in idx[b, t]]
                s = [0.5 * sum(float(qf[b, t, h, d]) * float(r[d]) for d in range(d_qk))
                     for r in rows]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                for d in range(d_v):
                    ref = sum(wi * float(r[d]) for wi, r in zip(w, rows)) / tot
                    assert abs(out[b, t, h, d] - ref) < 1e-12
                assert abs(lse[b, t, h] - (m + math.log(tot))) < 1e-12


def test_one_token_per_sequence_is_the_decode_case():
    rng = np.random.default_rng(72)
    kv = random_bits(rng, (3, 20, 8))
    q = random_bits(rng, (3, 4, 8))
    idx = np.stack([rng.choice(20, 7, replace=False) for _ in range(3)])
    o1, l1 = oracle.sparse_topk_attn(q[:, None], kv, idx[:, None], 5, 0.3)
    o2, l2 = oracle.sparse_topk_decode(q, kv, idx, 5, 0.3)
    assert np.array_equal(o1[:, 0], o2) and np.array_equal(l1[:, 0], l2)


def test_tokens_are_independent():
    """Swapping two tokens' queries and index lists swaps their outputs."""
    rng = np.random.default_rng(73)
    kv = random_bits(rng, (1, 30, 8))
    q = random_bits(rng, (1, 3, 2, 8))
    idx = np.stack([np.stack([rng.choice(30, 5, replace=False) for _ in range(3)])])
    out, lse = oracle.sparse_topk_attn(q, kv, idx, 8, 0.4)
    perm = [2, 0, 1]
    out_p, lse_p = oracle.sparse_topk_attn(q[:, perm], kv, idx[:, perm], 8, 0.4)
    assert np.array_equal(out_p, out[:, perm]) and np.array_equal(lse_p, lse[:, perm])
