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
