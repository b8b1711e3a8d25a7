"""Pins of the FP4 (E2M1) KV cache oracle -- CPU only."""

import numpy as np
import pytest

import oracle
from oracle import fp4, round_to_bf16_bits


def e2m1_value(code):
    """The format's definition: sign bit 3, exponent bits 2..1 with bias 1, mantissa
    bit 0; exponent field 0 is the subnormal m * 2^0 * 0.5."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if s else mag


def test_every_code_decodes_by_the_format_definition():
    codes = np.arange(16)
    assert np.array_equal(fp4.e2m1_decode(codes), [e2m1_value(int(c)) for c in codes])
    assert sorted(set(np.abs(fp4.e2m1_decode(codes)))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_encoding_is_the_nearest_value_ties_to_even_by_brute_force():
    vals = np.array([e2m1_value(c) for c in range(16)])
    grid = np.unique(np.concatenate([np.linspace(-6, 6, 2401), (vals[:-1] + vals[1:]) / 2,
                                     vals, [0.25, -0.25, 0.75, 5.0, -5.0]]))
    grid = grid[np.abs(grid) <= 6]
    got = fp4.e2m1_encode(grid)
    for x, c in zip(grid, got):
        d = np.abs(vals - x)
        best = [k for k in range(16) if d[k] == d.min()]
        if vals[best[0]] == 0 and 0 in best:
            assert c == 0, x                   # nearest value (or a tie with) zero: +0
            continue
        assert c in best, (x, c, best)
        if len(best) > 1:
            assert c % 2 == 0, (x, c, best)    # a tie goes to the even code


def test_scale_is_the_smallest_power_of_two_that_fits():
    for amax in [6.0, 6.0001, 3.0, 3.0001, 1e-30, 1e30, 0.7, 12.0]:
        e = fp4.scale_exponent(amax)
        assert amax <= 6.0 * 2.0 ** e and amax > 6.0 * 2.0 ** (e - 1)
    assert fp4.scale_exponent(0.0) == 0


def test_packing_puts_the_even_element_in_the_low_four_bits():
    codes = np.array([[1, 2, 7, 8, 15, 0]], np.uint8)
    packed = fp4.pack(codes)
    assert packed.tolist() == [[0x21, 0x87, 0x0F]]
    assert np.array_equal(fp4.unpack(packed), codes)


def test_quantisation_error_is_at_most_half_a_step_of_the_scaled_grid():
    rng = np.random.default_rng(50)
    x = rng.standard_normal((32, 64)) * np.exp(rng.uniform(-6, 6, (32, 1)))
    bits = round_to_bf16_bits(x)
    packed, scale = fp4.quantize_rows(bits)
    xs = oracle.widen(bits) / scale[:, None]
    assert np.all(np.abs(xs) <= 6.0) and np.all(np.max(np.abs(xs), axis=1) > 3.0)
    deq = fp4.e2m1_decode(fp4.unpack(packed))
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.abs(xs)
    hi = np.minimum(np.searchsorted(mags, a), 7)
    lo = np.maximum(hi - 1, 0)
    assert np.all(np.abs(np.abs(deq) - a) <= (mags[hi] - mags[lo]) / 2 + 1e-300)


def test_attention_over_fp4_cache_equals_bf16_layout_of_the_same_values():
    rng = np.random.default_rng(51)
    B, H, cap, D = 2, 3, 40, 16
    kc, ks = fp4.quantize_rows(round_to_bf16_bits(rng.standard_normal((B, H, cap, D)) * 2))
    vc, vs = fp4.quantize_rows(round_to_bf16_bits(rng.standard_normal((B, H, cap, D))))
    k_deq = round_to_bf16_bits(fp4.dequantize(kc, ks))
    v_deq = round_to_bf16_bits(fp4.dequantize(vc, vs))
    assert np.array_equal(oracle.widen(k_deq), fp4.dequantize(kc, ks))
    mask = (rng.uniform(size=(B, cap)) < 0.6).astype(np.int32)
    q = rng.standard_normal((B, H, D))
    a, la = oracle.decode_static_fp4(q, kc, vc, ks, vs, mask=mask, valid_len=[33, 40])
    b, lb = oracle.decode_static(q, k_deq, v_deq, mask=mask, valid_len=[33, 40])
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_append_quantises_the_new_row_and_rejects_positions_outside():
    rng = np.random.default_rng(52)
    B, H, cap, D = 2, 2, 6, 8
    kc = np.zeros((B, H, cap, D // 2), np.uint8)
    ks = np.ones((B, H, cap))
    kn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    vn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    mask = np.zeros((B, cap), np.int32)
    out = oracle.kv_append_fp4(kc, kc, ks, ks, kn, vn, [0, 5], mask)
    qk, sk = fp4.quantize_rows(kn)
    assert np.array_equal(out[0][0, :, 0], qk[0]) and np.array_equal(out[2][1, :, 5], sk[1])
    assert out[4][0].tolist() == [1, 0, 0, 0, 0, 0] and out[4][1, 5] == 1
    with pytest.raises(ValueError):
        oracle.kv_append_fp4(kc, kc, ks, ks, kn, vn, [6, 0])


# ------------------------------------------------- the sparse kernel's FP4 latent cache


def representable_latent_rows(rng, B, n, d):
    """Packed latent rows whose values are E2M1 values times a power of two, with a
    code of magnitude 6 in each row: quantising them gives back exactly these codes
    and scales (no -0 codes: zeros are stored as +0)."""
    nib = rng.integers(0, 16, size=(B, n, d)).astype(np.uint8)
    nib[nib == 8] = 0                              # -0 -> +0
    nib[..., 0] = 7 | (nib[..., 0] & 8)            # magnitude 6
    scale = np.exp2(rng.integers(-8, -2, size=(B, n))).astype(np.float64)
    return fp4.pack(nib), scale


def test_latent_append_fp4_round_trips_576_wide_rows_and_rejects_positions_outside():
    rng = np.random.default_rng(56)
    B, s_kv, d = 3, 7, 576
    codes0 = rng.integers(0, 256, size=(B, s_kv, d // 2)).astype(np.uint8)
    scale0 = np.full((B, s_kv), 0.5)
    new_codes, new_scale = representable_latent_rows(rng, B, 1, d)
    rows = round_to_bf16_bits(fp4.dequantize(new_codes[:, 0], new_scale[:, 0]))
    pos = np.array([6, 0, 2])
    codes, scale = oracle.latent_append_fp4(codes0, scale0, rows, pos)
    for b in range(B):
        assert np.array_equal(codes[b, pos[b]], new_codes[b, 0])
        assert scale[b, pos[b]] == new_scale[b, 0]
        others = np.arange(s_kv) != pos[b]
        assert np.array_equal(codes[b, others], codes0[b, others])
        assert np.array_equal(scale[b, others], scale0[b, others])
    for bad in ([0, 7, 1], [-1, 0, 1]):
        with pytest.raises(ValueError):
            oracle.latent_append_fp4(codes0, scale0, rows, np.array(bad))


def test_sparse_fp4_equals_bf16_sparse_over_the_dequantised_rows():
    rng = np.random.default_rng(57)
    B, s_q, h_q, s_kv, d, d_v, topk = 2, 2, 4, 40, 24, 16, 13
    codes, scale = representable_latent_rows(rng, B, s_kv, d)
    deq = fp4.dequantize(codes, scale)
    kv_bits = round_to_bf16_bits(deq)
    assert np.array_equal(oracle.widen(kv_bits), deq)
    q = rng.standard_normal((B, s_q, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, s_q, topk))
    a, la = oracle.sparse_topk_attn_fp4(q, codes, scale, idx, d_v, 0.3)
    b, lb = oracle.sparse_topk_attn(q, kv_bits, idx, d_v, 0.3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_sparse_fp4_over_equal_rows_is_that_row():
    rng = np.random.default_rng(58)
    B, s_kv, d, d_v, h_q, topk = 1, 9, 32, 20, 3, 6
    row_codes, row_scale = representable_latent_rows(rng, 1, 1, d)
    codes = np.broadcast_to(row_codes, (B, s_kv, d // 2)).copy()
    scale = np.full((B, s_kv), row_scale[0, 0])
    q = rng.standard_normal((B, 1, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, 1, topk))
    out, lse = oracle.sparse_topk_attn_fp4(q, codes, scale, idx, d_v, 0.5)
    row = fp4.dequantize(row_codes[0, 0], row_scale[0, 0])
    for h in range(h_q):
        assert np.allclose(out[0, 0, h], row[:d_v], rtol=0, atol=1e-12)
        assert np.isclose(lse[0, 0, h], 0.5 * q[0, 0, h] @ row + np.log(topk), rtol=0,
                          atol=1e-12)


def test_sparse_fp4_scale_acts_on_whole_rows():
    rng = np.random.default_rng(59)
    B, s_kv, d, d_v, h_q, topk = 2, 30, 40, 32, 5, 11
    codes, scale = representable_latent_rows(rng, B, s_kv, d)
    q = rng.standard_normal((B, 1, h_q, d))
    idx = rng.integers(0, s_kv, size=(B, 1, topk))
    o1, l1 = oracle.sparse_topk_attn_fp4(q, codes, scale, idx, d_v, 0.2)
    o2, l2 = oracle.sparse_topk_attn_fp4(q / 2, codes, scale * 2, idx, d_v, 0.2)
    assert np.allclose(o2, 2 * o1, rtol=1e-12, atol=0)
    assert np.allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_sparse_fp4_rejects_out_of_range_indices():
    codes = np.zeros((1, 5, 4), dtype=np.uint8)
    scale = np.ones((1, 5))
    q = np.ones((1, 1, 2, 8))
    for bad in (5, -1):
        with pytest.raises(ValueError):
            oracle.sparse_topk_attn_fp4(q, codes, scale, np.array([[[0, bad]]]), 4, 1.0)


# ------------------------------------------------------------------ paged FP4 pool


def _small_pool_fp4(rng, lengths, bs, Hkv, D):
    """A pool holding the E2M1-quantised rows of random bf16 K/V, its table and offsets."""
    need = [-(-L // bs) for L in lengths]
    nb = sum(need) + 3
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((len(lengths), max(need)), -1, np.int32)
    at = 0
    for q, n in enumerate(need):
        tables[q, :n] = perm[at:at + n]
        at += n
    seq_lens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    kc, ks = fp4.quantize_rows(round_to_bf16_bits(rng.standard_normal((nb, bs, Hkv, D)) * 2))
    vc, vs = fp4.quantize_rows(round_to_bf16_bits(rng.standard_normal((nb, bs, Hkv, D))))
    return kc, vc, ks, vs, tables, seq_lens


def test_paged_fp4_decode_equals_bf16_paged_decode_of_the_same_values():
    rng = np.random.default_rng(61)
    lengths, bs, Hkv, D, Hq = [5, 16, 33], 8, 2, 16, 4
    kc, vc, ks, vs, tables, seq_lens = _small_pool_fp4(rng, lengths, bs, Hkv, D)
    k_deq = round_to_bf16_bits(fp4.dequantize(kc, ks))
    v_deq = round_to_bf16_bits(fp4.dequantize(vc, vs))
    assert np.array_equal(oracle.widen(v_deq), fp4.dequantize(vc, vs))
    q = round_to_bf16_bits(rng.standard_normal((3, Hq, D)))
    a, la = oracle.decode_paged_fp4(q, kc, vc, ks, vs, tables, seq_lens)
    b, lb = oracle.decode_paged(q, k_deq, v_deq, tables, seq_lens)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_paged_fp4_decode_equals_static_fp4_decode_of_the_same_rows():
    rng = np.random.default_rng(62)
    lengths, bs, Hkv, D, group = [7, 12], 4, 2, 8, 2
    kc, vc, ks, vs, tables, seq_lens = _small_pool_fp4(rng, lengths, bs, Hkv, D)
    q = rng.standard_normal((2, Hkv * group, D))
    out, lse = oracle.decode_paged_fp4(q, kc, vc, ks, vs, tables, seq_lens)
    cap = max(lengths)
    for b, L in enumerate(lengths):
        t = np.arange(L)
        phys, slot = tables[b, t // bs], t % bs
        skc = np.zeros((1, Hkv * group, cap, D // 2), np.uint8)
        svc = np.zeros_like(skc)
        sks = np.ones((1, Hkv * group, cap))
        svs = np.ones_like(sks)
        for h in range(Hkv * group):
            skc[0, h, :L] = kc[phys, slot, h // group]
            svc[0, h, :L] = vc[phys, slot, h // group]
            sks[0, h, :L] = ks[phys, slot, h // group]
            svs[0, h, :L] = vs[phys, slot, h // group]
        o2, l2 = oracle.decode_static_fp4(q[b:b + 1], skc, svc, sks, svs, valid_len=[L])
        assert np.allclose(out[b], o2[0], rtol=0, atol=1e-13)
        assert np.allclose(lse[b], l2[0], rtol=0, atol=1e-13)


def test_paged_append_fp4_places_the_new_token_at_the_last_position():
    rng = np.random.default_rng(63)
    lengths, bs, Hkv, D = [1, 9, 16], 8, 2, 16
    kc, vc, ks, vs, tables, seq_lens = _small_pool_fp4(rng, lengths, bs, Hkv, D)
    kn = round_to_bf16_bits(rng.standard_normal((3, Hkv, D)) * 5)
    vn = round_to_bf16_bits(rng.standard_normal((3, Hkv, D)))
    kc2, vc2, ks2, vs2 = oracle.paged_append_fp4(kc, vc, ks, vs, kn, vn, tables, seq_lens)
    qk, sk = fp4.quantize_rows(kn)
    qv, sv = fp4.quantize_rows(vn)
    changed = np.zeros(kc.shape[:2], bool)
    for b, L in enumerate(lengths):
        p, s = tables[b, (L - 1) // bs], (L - 1) % bs
        assert np.array_equal(kc2[p, s], qk[b]) and np.array_equal(vc2[p, s], qv[b])
        assert np.array_equal(ks2[p, s], sk[b]) and np.array_equal(vs2[p, s], sv[b])
        changed[p, s] = True
    assert np.array_equal(kc2[~changed], kc[~changed]) and np.array_equal(vs2[~changed], vs[~changed])
    with pytest.raises(ValueError):
        oracle.paged_append_fp4(kc, vc, ks, vs, kn, vn, tables,
                                np.array([0, 1, 1, 17], np.int32))
