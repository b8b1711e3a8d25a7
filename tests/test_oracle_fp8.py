"""Pins of the FP8 KV-cache oracle (CPU): the E4M3 code table and rounding against
torch's float8_e4m3fn, the scale rule, the quantisation error bound, and attention
over the FP8 cache equal to attention over the same values in the bf16 layout."""

import numpy as np
import pytest
import torch

import oracle
from oracle import round_to_bf16_bits


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_every_code_decodes_like_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encoding_rounds_to_nearest_even_like_torch():
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2                        # exact ties
    rng = np.random.default_rng(40)
    rand = rng.uniform(0, 448, 4000)
    tiny = rng.uniform(0, 2.0 ** -6, 2000)                   # subnormal range
    x = np.concatenate([grid, mids, rand, tiny])
    x = np.concatenate([x, -x])
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # zero results are always the +0 code here; torch keeps the sign of a zero
    zero = oracle.e4m3_decode(ours) == 0
    assert np.array_equal(ours[~zero], ref[~zero])
    assert np.all(torch_decode(ref[zero]) == 0)
    assert np.all(ours[zero] == 0)


def test_scale_is_the_smallest_power_of_two_that_fits():
    rng = np.random.default_rng(41)
    amax = np.concatenate([rng.uniform(1e-30, 1e30, 500) ** rng.uniform(0, 1, 500),
                           [448.0, 449.0, 224.0, 224.0001, 1.0, 3.0e38, 1e-38]])
    for a in amax:
        e = oracle.scale_exponent(a)
        assert a <= 448.0 * 2.0 ** e
        assert a > 448.0 * 2.0 ** (e - 1)
    assert oracle.scale_exponent(0.0) == 0


def test_quantisation_error_is_at_most_half_a_grid_step():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    bits = round_to_bf16_bits(x)
    codes, scale = oracle.quantize_rows(bits)
    xs = oracle.widen(bits) / scale[:, None]
    assert np.all(np.abs(xs) <= 448.0) and np.all(np.max(np.abs(xs), axis=1) > 224.0)
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    deq = oracle.e4m3_decode(codes)
    a = np.abs(xs)
    hi = np.minimum(np.searchsorted(grid, a), len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    step = grid[hi] - grid[lo]
    assert np.all(np.abs(deq - xs) <= step / 2 + 1e-300)


def test_attention_over_fp8_cache_equals_bf16_layout_of_the_same_values():
    rng = np.random.default_rng(43)
    B, H, cap, D = 2, 3, 50, 16
    k_bits = round_to_bf16_bits(rng.standard_normal((B, H, cap, D)) * 3)
    v_bits = round_to_bf16_bits(rng.standard_normal((B, H, cap, D)))
    kc, ks = oracle.quantize_rows(k_bits)
    vc, vs = oracle.quantize_rows(v_bits)
    # the dequantised values are bf16 numbers: the same cache in the bf16 layout
    k_deq = round_to_bf16_bits(oracle.e4m3_decode(kc) * ks[..., None])
    v_deq = round_to_bf16_bits(oracle.e4m3_decode(vc) * vs[..., None])
    assert np.array_equal(oracle.widen(k_deq), oracle.e4m3_decode(kc) * ks[..., None])
    mask = (rng.uniform(size=(B, cap)) < 0.7).astype(np.int32)
    q = rng.standard_normal((B, H, D))
    a, la = oracle.decode_static_fp8(q, kc, vc, ks, vs, mask=mask, valid_len=[40, 50])
    b, lb = oracle.decode_static(q, k_deq, v_deq, mask=mask, valid_len=[40, 50])
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_append_quantises_the_new_row_and_rejects_positions_outside():
    rng = np.random.default_rng(44)
    B, H, cap, D = 2, 2, 8, 16
    kc = np.zeros((B, H, cap, D), np.uint8)
    vc = np.zeros((B, H, cap, D), np.uint8)
    ks = np.ones((B, H, cap))
    vs = np.ones((B, H, cap))
    kn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    vn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    mask = np.zeros((B, cap), np.int32)
    kc2, vc2, ks2, vs2, m2 = oracle.kv_append_fp8(kc, vc, ks, vs, kn, vn, [3, 7], mask)
    qk, sk = oracle.quantize_rows(kn)
    assert np.array_equal(kc2[0, :, 3], qk[0]) and np.array_equal(ks2[1, :, 7], sk[1])
    assert m2[0].tolist() == [0, 0, 0, 1, 0, 0, 0, 0] and m2[1, 7] == 1
    assert np.array_equal(kc2[0, :, :3], kc[0, :, :3])
    with pytest.raises(ValueError):
        oracle.kv_append_fp8(kc, vc, ks, vs, kn, vn, [8, 0])


# ------------------------------------------------------------------ paged FP8 pool


def _small_pool(rng, lengths, bs, Hkv, D):
    """A pool holding the quantised rows of random bf16 K/V, its table and offsets."""
    need = [-(-L // bs) for L in lengths]
    nb = sum(need) + 3
    perm = rng.permutation(nb).astype(np.int32)
    cols = max(need)
    tables = np.full((len(lengths), cols), -1, np.int32)
    at = 0
    for q, n in enumerate(need):
        tables[q, :n] = perm[at:at + n]
        at += n
    seq_lens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    k_bits = round_to_bf16_bits(rng.standard_normal((nb, bs, Hkv, D)) * 2)
    v_bits = round_to_bf16_bits(rng.standard_normal((nb, bs, Hkv, D)))
    kc, ks = oracle.quantize_rows(k_bits)
    vc, vs = oracle.quantize_rows(v_bits)
    return kc, vc, ks, vs, tables, seq_lens


def test_paged_fp8_decode_equals_bf16_paged_decode_of_the_same_values():
    """The FP8 pool's attention is decode_paged (pinned on its own) over a bf16 pool
    holding the dequantised values, bit for bit."""
    rng = np.random.default_rng(45)
    lengths, bs, Hkv, D, Hq = [5, 16, 33], 8, 2, 16, 4
    kc, vc, ks, vs, tables, seq_lens = _small_pool(rng, lengths, bs, Hkv, D)
    k_deq = round_to_bf16_bits(oracle.e4m3_decode(kc) * ks[..., None])
    v_deq = round_to_bf16_bits(oracle.e4m3_decode(vc) * vs[..., None])
    assert np.array_equal(oracle.widen(v_deq), oracle.e4m3_decode(vc) * vs[..., None])
    q = round_to_bf16_bits(rng.standard_normal((3, Hq, D)))
    a, la = oracle.decode_paged_fp8(q, kc, vc, ks, vs, tables, seq_lens)
    b, lb = oracle.decode_paged(q, k_deq, v_deq, tables, seq_lens)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_paged_fp8_decode_equals_static_fp8_decode_of_the_same_rows():
    """Laying each sequence's rows out in a static buffer (GQA: KV head h // group)
    gives the static FP8 oracle's result."""
    rng = np.random.default_rng(46)
    lengths, bs, Hkv, D, group = [7, 12], 4, 2, 8, 2
    kc, vc, ks, vs, tables, seq_lens = _small_pool(rng, lengths, bs, Hkv, D)
    q = rng.standard_normal((2, Hkv * group, D))
    out, lse = oracle.decode_paged_fp8(q, kc, vc, ks, vs, tables, seq_lens)
    cap = max(lengths)
    for b, L in enumerate(lengths):
        t = np.arange(L)
        phys, slot = tables[b, t // bs], t % bs
        skc = np.zeros((1, Hkv * group, cap, D), np.uint8)
        svc = np.zeros_like(skc)
        sks = np.ones((1, Hkv * group, cap))
        svs = np.ones_like(sks)
        for h in range(Hkv * group):
            skc[0, h, :L] = kc[phys, slot, h // group]
            svc[0, h, :L] = vc[phys, slot, h // group]
            sks[0, h, :L] = ks[phys, slot, h // group]
            svs[0, h, :L] = vs[phys, slot, h // group]
        o2, l2 = oracle.decode_static_fp8(q[b:b + 1], skc, svc, sks, svs, valid_len=[L])
        assert np.allclose(out[b], o2[0], rtol=0, atol=1e-13)
        assert np.allclose(lse[b], l2[0], rtol=0, atol=1e-13)


def test_paged_append_places_the_new_token_at_the_last_position():
    rng = np.random.default_rng(47)
    lengths, bs, Hkv, D = [1, 9, 16], 8, 2, 16
    kc, vc, ks, vs, tables, seq_lens = _small_pool(rng, lengths, bs, Hkv, D)
    kn = round_to_bf16_bits(rng.standard_normal((3, Hkv, D)) * 5)
    vn = round_to_bf16_bits(rng.standard_normal((3, Hkv, D)))
    kc2, vc2, ks2, vs2 = oracle.paged_append_fp8(kc, vc, ks, vs, kn, vn, tables, seq_lens)
    qk, sk = oracle.quantize_rows(kn)
    qv, sv = oracle.quantize_rows(vn)
    changed = np.zeros(kc.shape[:2], bool)
    for b, L in enumerate(lengths):
        p, s = tables[b, (L - 1) // bs], (L - 1) % bs     # token L-1: block, slot
        assert np.array_equal(kc2[p, s], qk[b]) and np.array_equal(vc2[p, s], qv[b])
        assert np.array_equal(ks2[p, s], sk[b]) and np.array_equal(vs2[p, s], sv[b])
        changed[p, s] = True
    assert np.array_equal(kc2[~changed], kc[~changed]) and np.array_equal(vs2[~changed], vs[~changed])
    with pytest.raises(ValueError):
        oracle.paged_append_fp8(kc, vc, ks, vs, kn, vn, tables,
                                np.array([0, 1, 1, 17], np.int32))   # a length-0 sequence


# ------------------------------------------------- the sparse kernel's FP8 latent cache


def representable_latent_rows(rng, B, n, d):
    """Latent rows whose values are E4M3 values times a power of two, with one code of
    magnitude above 224 per row: quantising them must give back exactly these codes
    and scales (the scale rule picks that exponent; no -0 codes)."""
    codes = rng.integers(0, 256, size=(B, n, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E          # no NaN codes
    codes[codes == 0x80] = 0x00                   # zeros as +0
    codes[..., 0] = 0x7A | (codes[..., 0] & 0x80)  # 0x7A = 320 > 224
    scale = np.exp2(rng.integers(-10, -4, size=(B, n))).astype(np.float64)
    return codes, scale


def test_latent_append_round_trips_576_wide_rows_and_rejects_positions_outside():
    rng = np.random.default_rng(46)
    B, s_kv, d = 3, 7, 576
    codes0 = rng.integers(0, 0x70, size=(B, s_kv, d)).astype(np.uint8)
    scale0 = np.full((B, s_kv), 0.25)
    new_codes, new_scale = representable_latent_rows(rng, B, 1, d)
    rows = round_to_bf16_bits(oracle.e4m3_decode(new_codes[:, 0]) * new_scale[:, :1])
    pos = np.array([0, 6, 3])
    codes, scale = oracle.latent_append_fp8(codes0, scale0, rows, pos)
    for b in range(B):
        assert np.array_equal(codes[b, pos[b]], new_codes[b, 0])
        assert scale[b, pos[b]] == new_scale[b, 0]
        others = np.arange(s_kv) != pos[b]
        assert np.array_equal(codes[b, others], codes0[b, others])
        assert np.array_equal(scale[b, others], scale0[b, others])
    with pytest.raises(ValueError):
        oracle.latent_append_fp8(codes0, scale0, rows, np.array([0, 7, 1]))
    with pytest.raises(ValueError):
        oracle.latent_append_fp8(codes0, scale0, rows, np.array([-1, 0, 1]))


def test_sparse_fp8_equals_bf16_sparse_over_the_dequantised_rows():
    rng = np.random.default_rng(47)
    B, s_q, h_q, s_kv, d, d_v, topk = 2, 2, 4, 40, 24, 16, 13
    codes, scale = representable_latent_rows(rng, B, s_kv, d)
    kv_bits = round_to_bf16_bits(oracle.e4m3_decode(codes) * scale[..., None])
    assert np.array_equal(oracle.widen(kv_bits), oracle.e4m3_decode(codes) * scale[..., None])
    q = rng.standard_normal((B, s_q, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, s_q, topk))
    a, la = oracle.sparse_topk_attn_fp8(q, codes, scale, idx, d_v, 0.3)
    b, lb = oracle.sparse_topk_attn(q, kv_bits, idx, d_v, 0.3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_sparse_fp8_over_equal_rows_is_that_row():
    """Every gathered row the same: every head's output is the dequantised row's first
    d_v values and its log-sum-exp the common score plus ln(topk)."""
    rng = np.random.default_rng(48)
    B, s_kv, d, d_v, h_q, topk = 1, 9, 32, 20, 3, 6
    row_codes, row_scale = representable_latent_rows(rng, 1, 1, d)
    codes = np.broadcast_to(row_codes, (B, s_kv, d)).copy()
    scale = np.full((B, s_kv), row_scale[0, 0])
    q = rng.standard_normal((B, 1, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, 1, topk))
    out, lse = oracle.sparse_topk_attn_fp8(q, codes, scale, idx, d_v, 0.5)
    row = oracle.e4m3_decode(row_codes[0, 0]) * row_scale[0, 0]
    for h in range(h_q):
        assert np.allclose(out[0, 0, h], row[:d_v], rtol=0, atol=1e-12)
        assert np.isclose(lse[0, 0, h], 0.5 * q[0, 0, h] @ row + np.log(topk), rtol=0,
                          atol=1e-12)


def test_sparse_fp8_scale_acts_on_whole_rows():
    """Doubling every row scale while halving q leaves the scores unchanged, so the
    output doubles (the value columns double) and the log-sum-exp is unchanged: a
    scale applied to part of a row, or not at all, breaks this."""
    rng = np.random.default_rng(49)
    B, s_kv, d, d_v, h_q, topk = 2, 30, 40, 32, 5, 11
    codes, scale = representable_latent_rows(rng, B, s_kv, d)
    q = rng.standard_normal((B, 1, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, 1, topk))
    o1, l1 = oracle.sparse_topk_attn_fp8(q, codes, scale, idx, d_v, 0.2)
    o2, l2 = oracle.sparse_topk_attn_fp8(q / 2, codes, scale * 2, idx, d_v, 0.2)
    assert np.allclose(o2, 2 * o1, rtol=1e-12, atol=0)
    assert np.allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_sparse_fp8_rejects_out_of_range_indices():
    codes = np.zeros((1, 5, 8), dtype=np.uint8)
    scale = np.ones((1, 5))
    q = np.ones((1, 1, 2, 8))
    for bad in (5, -1):
        with pytest.raises(ValueError):
            oracle.sparse_topk_attn_fp8(q, codes, scale, np.array([[[0, bad]]]), 4, 1.0)
