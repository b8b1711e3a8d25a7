"""Pins of the static-buffer oracle (append + masked decode attention) -- CPU only.

Each test checks the oracle against something other than itself: values the
pages print, closed forms, invariants, a library routine on a special case, or
brute force on tiny inputs.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import round_to_bf16_bits, widen
from conftest import bits, npy

import workloads


def sdpa_f64(q, K, V, keep, scale):
    """torch's scaled_dot_product_attention in float64 on one query row."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64)).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64)).view(1, 1, V.shape[0], -1)
    bias = torch.where(torch.from_numpy(np.asarray(keep, dtype=bool)),
                       torch.tensor(0.0, dtype=torch.float64),
                       torch.tensor(-math.inf, dtype=torch.float64)).view(1, 1, 1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=bias,
                                                         scale=scale)
    return out.view(-1).numpy()


def random_bf16(rng, shape, std=1.0):
    return round_to_bf16_bits(rng.standard_normal(shape) * std)


# ----------------------------------------------------------------- closed forms


def test_bf16_widen_exact():
    # 1.0, -2.0, 0.5, smallest normal, +inf, the bf16 of pi (0x4049 = 3.140625)
    u = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x7F80, 0x4049], dtype=np.uint16)
    expect = [1.0, -2.0, 0.5, 2.0 ** -126, math.inf, 3.140625]
    assert widen(u).tolist() == expect
    assert round_to_bf16_bits(np.array([1.0, math.pi, -2.0])).tolist() == [0x3F80, 0x4049, 0xC000]
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert round_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert round_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_two_row_hand_example():
    # D = 1, scale = 1, q = 1, K = [0, ln 3], V = [1, 5]:
    # weights 1/4, 3/4 -> out = 1/4 + 15/4 = 4; lse = ln(1 + 3) = ln 4.
    # ln 3 is not a bf16 value, so K is built as float bits of the rounded value and
    # the expectation uses that rounded value.
    k1 = round_to_bf16_bits(np.array([math.log(3.0)]))[0]
    k1v = float(widen(np.array([k1], dtype=np.uint16))[0])
    K = np.array([0x0000, k1], dtype=np.uint16).reshape(1, 1, 2, 1)
    V = round_to_bf16_bits(np.array([1.0, 5.0])).reshape(1, 1, 2, 1)
    out, lse = oracle.decode_static(np.ones((1, 1, 1)), K, V, valid_len=[2], scale=1.0)
    w1 = math.exp(k1v) / (1.0 + math.exp(k1v))
    assert out[0, 0, 0] == pytest.approx((1 - w1) * 1.0 + w1 * 5.0, abs=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(1.0 + math.exp(k1v)), abs=1e-14)
    # and with the exact ln 3 the textbook numbers come out
    assert (1 - 0.75) * 1 + 0.75 * 5 == 4.0


def test_single_row_returns_that_row_exactly():
    rng = np.random.default_rng(0)
    B, H, cap, D = 2, 3, 16, 8
    K = random_bf16(rng, (B, H, cap, D))
    V = random_bf16(rng, (B, H, cap, D))
    q = rng.standard_normal((B, H, D))
    out, lse = oracle.decode_static(q, K, V, valid_len=[1, 1], scale=0.3)
    assert np.array_equal(out, widen(V[:, :, 0, :]))
    expect_lse = 0.3 * np.einsum("bhd,bhd->bh", widen(K[:, :, 0, :]), q)
    assert np.allclose(lse, expect_lse, rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_valid_rows():
    rng = np.random.default_rng(1)
    B, H, cap, D = 1, 2, 32, 4
    K = random_bf16(rng, (B, H, cap, D))
    V = random_bf16(rng, (B, H, cap, D))
    L = 13
    out, lse = oracle.decode_static(np.zeros((B, H, D)), K, V, valid_len=[L])
    assert np.allclose(out, widen(V[:, :, :L, :]).mean(axis=2), atol=1e-15)
    assert np.allclose(lse, math.log(L), atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    cap, D = 10, 16
    row = random_bf16(rng, (D,))
    K = np.broadcast_to(row, (1, 1, cap, D)).copy()
    V = random_bf16(rng, (1, 1, cap, D))
    q = rng.standard_normal((1, 1, D))
    mask = np.array([[1, 0, 1, 1, 0, 1, 0, 0, 1, 1]])
    out, lse = oracle.decode_static(q, K, V, mask=mask)
    rows = np.flatnonzero(mask[0])
    s = (widen(row) @ q[0, 0]) / math.sqrt(D)
    assert np.allclose(out[0, 0], widen(V[0, 0, rows]).mean(axis=0), atol=1e-15)
    assert lse[0, 0] == pytest.approx(s + math.log(len(rows)), abs=1e-13)


def test_fully_masked_sequence_is_zero_with_minus_inf_lse():
    rng = np.random.default_rng(3)
    K = random_bf16(rng, (2, 1, 4, 2))
    V = random_bf16(rng, (2, 1, 4, 2))
    out, lse = oracle.decode_static(rng.standard_normal((2, 1, 2)), K, V,
                                    mask=np.array([[0, 0, 0, 0], [1, 1, 0, 0]]))
    assert np.all(out[0] == 0) and lse[0, 0] == -math.inf
    assert np.isfinite(lse[1, 0])


# ------------------------------------------------------------ library routine


@pytest.mark.parametrize("D,L,cap", [(64, 103, 1152), (128, 777, 1024), (8, 5, 8)])
def test_matches_torch_sdpa_float64(D, L, cap):
    rng = np.random.default_rng(D + L)
    K = random_bf16(rng, (1, 2, cap, D))
    V = random_bf16(rng, (1, 2, cap, D))
    q = rng.standard_normal((1, 2, D))
    mask = (rng.random((1, cap)) < 0.7).astype(np.int32)
    mask[0, 0] = 1
    out, _ = oracle.decode_static(q, K, V, mask=mask, valid_len=[L])
    keep = (mask[0] != 0) & (np.arange(cap) < L)
    for h in range(2):
        ref = sdpa_f64(q[0, h], widen(K[0, h]), widen(V[0, h]), keep, 1.0 / math.sqrt(D))
        assert np.max(np.abs(out[0, h] - ref)) < 1e-12


def test_brute_force_every_mask_tiny():
    """cap = 6: all 64 masks x several valid lengths x D in {1, 2, 8} vs SDPA."""
    rng = np.random.default_rng(4)
    cap = 6
    for D in (1, 2, 8):
        K = random_bf16(rng, (1, 1, cap, D), std=2.0)
        V = random_bf16(rng, (1, 1, cap, D))
        q = rng.standard_normal((1, 1, D))
        for m in itertools.product([0, 1], repeat=cap):
            mask = np.array([m], dtype=np.int32)
            for L in (0, 1, 3, cap):
                out, lse = oracle.decode_static(q, K, V, mask=mask, valid_len=[L], scale=0.7)
                keep = (mask[0] != 0) & (np.arange(cap) < L)
                if not keep.any():
                    assert np.all(out == 0) and lse[0, 0] == -math.inf
                    continue
                ref = sdpa_f64(q[0, 0], widen(K[0, 0]), widen(V[0, 0]), keep, 0.7)
                assert np.max(np.abs(out[0, 0] - ref)) < 1e-13
                s = 0.7 * (widen(K[0, 0, keep]) @ q[0, 0])
                assert lse[0, 0] == pytest.approx(math.log(np.sum(np.exp(s))), abs=1e-12)


# ------------------------------------------------------------------ invariants


@pytest.mark.parametrize("poison", ["sigma100", "inf", "nan"])
def test_garbage_outside_attended_rows_never_matters(poison):
    case = workloads.static_case(2, 3, 16, 40, [7, 29], seed=5, mask_density=0.8)
    K, V = bits(case.k_cache), bits(case.v_cache)
    mask, valid = npy(case.mask), npy(case.valid_len)
    out0, lse0 = oracle.decode_static(npy(case.q), K, V, mask, valid)
    rng = np.random.default_rng(6)
    K2, V2 = K.copy(), V.copy()
    for b, L in enumerate(case.lengths):
        dead = np.ones(40, dtype=bool)
        dead[:L] = mask[b, :L] == 0
        n = int(dead.sum()) * 3 * 16
        if poison == "sigma100":
            junk = random_bf16(rng, (n,), std=100.0)
        elif poison == "inf":
            junk = np.where(rng.random(n) < 0.5, 0x7F80, 0xFF80).astype(np.uint16)
        else:
            junk = np.full(n, 0x7FC0, dtype=np.uint16)
        K2[b][:, dead, :] = junk.reshape(3, -1, 16)
        V2[b][:, dead, :] = junk.reshape(3, -1, 16)[:, ::-1, :]
    out1, lse1 = oracle.decode_static(npy(case.q), K2, V2, mask, valid)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_permuting_attended_rows_leaves_output_unchanged():
    case = workloads.static_case(1, 2, 32, 64, [50], seed=7)
    K, V, q = bits(case.k_cache), bits(case.v_cache), npy(case.q)
    out0, lse0 = oracle.decode_static(q, K, V, valid_len=[50])
    perm = np.random.default_rng(8).permutation(50)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, :50] = K[:, :, perm]
    V2[:, :, :50] = V[:, :, perm]
    out1, lse1 = oracle.decode_static(q, K2, V2, valid_len=[50])
    assert np.allclose(out0, out1, rtol=0, atol=1e-14)
    assert np.allclose(lse0, lse1, rtol=0, atol=1e-13)


def test_right_slot_mask_form_equals_contiguous_form():
    """The NPU generate form [history..., 0...0, current] attends the same row set.

    Moving the current token's K/V from the last slot to the next free slot and
    using a contiguous mask must give the same result.
    """
    rng = np.random.default_rng(9)
    cap, D, hist = 16, 8, 5
    K = random_bf16(rng, (1, 1, cap, D))
    V = random_bf16(rng, (1, 1, cap, D))
    q = rng.standard_normal((1, 1, D))
    right = np.zeros((1, cap), dtype=np.int32)
    right[0, :hist] = 1
    right[0, cap - 1] = 1
    out_r, lse_r = oracle.decode_static(q, K, V, mask=right)
    K2, V2 = K.copy(), V.copy()
    K2[0, 0, hist] = K[0, 0, cap - 1]
    V2[0, 0, hist] = V[0, 0, cap - 1]
    out_c, lse_c = oracle.decode_static(q, K2, V2, valid_len=[hist + 1])
    assert np.allclose(out_r, out_c, rtol=0, atol=1e-14)
    assert np.allclose(lse_r, lse_c, rtol=0, atol=1e-13)


# -------------------------------------------------------- printed progression


def test_mask_progression_printed_on_the_page(golden_dir):
    """4-token prompt in a 1152-row buffer: 4, 5, ..., 103 valid rows (append then attend)."""
    g = json.load(open(os.path.join(golden_dir, "mask_progression.json")))
    cap = g["capacity"]
    assert cap == g["max_prompt_len"] + g["min_response_len"]
    P = g["prompt_tokens"]
    rng = np.random.default_rng(10)
    H, D = 2, 4
    K = np.zeros((1, H, cap, D), dtype=np.uint16)
    V = np.zeros((1, H, cap, D), dtype=np.uint16)
    K[0, :, :P] = random_bf16(rng, (H, P, D))
    V[0, :, :P] = random_bf16(rng, (H, P, D))
    mask = np.zeros((1, cap), dtype=np.int32)
    mask[0, :P] = 1
    printed = {p["generated_token"]: p for p in g["points"]}
    stored = P
    for n in range(1, 101):
        if n >= 2:
            # the input of step n is token n-1; its K/V go into the next free row
            kn, vn = random_bf16(rng, (1, H, D)), random_bf16(rng, (1, H, D))
            before_K = K.copy()
            K, V, mask = oracle.kv_append(K, V, kn, vn, [stored], mask)
            assert np.array_equal(K[0, :, stored], kn[0])
            untouched = np.ones(cap, dtype=bool)
            untouched[stored] = False
            assert np.array_equal(K[:, :, untouched], before_K[:, :, untouched])
            stored += 1
        L = int(mask.sum())
        assert L == n + 3 == stored
        if n in printed:
            assert L == printed[n]["valid_rows"]
            assert cap - L == printed[n]["padding_rows"]
        q = rng.standard_normal((1, H, D))
        by_mask, _ = oracle.decode_static(q, K, V, mask=mask)
        by_len, _ = oracle.decode_static(q, K, V, valid_len=[L])
        assert np.array_equal(by_mask, by_len)


def test_append_rejects_positions_outside_the_buffer():
    K = np.zeros((1, 1, 4, 2), dtype=np.uint16)
    new = np.ones((1, 1, 2), dtype=np.uint16)
    for pos in (-1, 4, 99):
        with pytest.raises(ValueError):
            oracle.kv_append(K, K, new, new, [pos])
    K2, _, _ = oracle.kv_append(K, K, new, new, [3])
    assert K2[0, 0, 3].tolist() == [1, 1] and K2[0, 0, :3].sum() == 0


def test_valid_length_outside_capacity_is_rejected():
    K = np.zeros((1, 1, 4, 2), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.decode_static(np.zeros((1, 1, 2)), K, K, valid_len=[5])
    with pytest.raises(ValueError):
        oracle.decode_static(np.zeros((1, 1, 2)), K, K)


# ------------------------------------------- prefill -> generate copy and trim


def _prefill_generate(rng, B, H, D, S_src, S_dst, lengths, n_tensors=2):
    src = [random_bf16(rng, (B, H, S_src, D)) for _ in range(n_tensors)]
    # the generate buffers start with garbage, NaN and Inf in every row
    dst = [random_bf16(rng, (B, H, S_dst, D), std=100.0) for _ in range(n_tensors)]
    for d in dst:
        d[:, :, ::7] = 0x7FC0   # NaN
        d[:, :, 3::11] = 0x7F80  # +Inf
    return src, dst


def test_copy_then_masked_attention_equals_attention_over_the_prompt(golden_dir):
    """The page's hand-over: prefill capacity 1024, generate capacity 1152, a prompt of
    4 tokens copied to rows [0:4]; the generate model then attends exactly the
    prompt rows (mask with 4 ones), whatever its buffer held before."""
    g = json.load(open(os.path.join(golden_dir, "mask_progression.json")))
    S_dst = g["capacity"]
    S_src = g["max_prompt_len"]
    rng = np.random.default_rng(30)
    B, H, D = 2, 2, 8
    lengths = [g["prompt_tokens"], 37]
    src, dst = _prefill_generate(rng, B, H, D, S_src, S_dst, lengths)
    mask0 = np.ones((B, S_dst), dtype=np.int32)
    new_dst, mask = oracle.copy_kvcache(src, dst, lengths, mask0)
    assert mask.sum(axis=1).tolist() == lengths
    q = rng.standard_normal((B, H, D))
    got, got_lse = oracle.decode_static(q, new_dst[0], new_dst[1], mask=mask)
    want, want_lse = oracle.decode_static(q, src[0], src[1], valid_len=lengths)
    assert np.array_equal(got, want) and np.array_equal(got_lse, want_lse)
    # rows at and after the length keep what the generate buffer held
    for d_old, d_new in zip(dst, new_dst):
        for b, n in enumerate(lengths):
            assert np.array_equal(d_new[b, :, n:], d_old[b, :, n:])


def test_copy_pairs_tensors_in_order_and_zero_length_copies_nothing():
    rng = np.random.default_rng(31)
    src, dst = _prefill_generate(rng, 1, 1, 8, 16, 20, [16], n_tensors=3)
    new_dst, _ = oracle.copy_kvcache(src, dst, [16])
    q = rng.standard_normal((1, 1, 8))
    for i in range(3):
        # tensor i of the generate model now answers like tensor i of the prefill model
        a, _ = oracle.decode_static(q, new_dst[i], new_dst[(i + 1) % 3], valid_len=[16])
        b, _ = oracle.decode_static(q, src[i], src[(i + 1) % 3], valid_len=[16])
        assert np.array_equal(a, b)
    same, _ = oracle.copy_kvcache(src, dst, [0])
    assert all(np.array_equal(x, y) for x, y in zip(same, dst))


def test_copy_then_generate_continues_the_printed_progression(golden_dir):
    """After the copy of a 4-token prompt, appends give 5, 6, ... valid rows (the page's
    4 -> 5 -> ... progression continues from the copied state)."""
    g = json.load(open(os.path.join(golden_dir, "mask_progression.json")))
    S_dst, S_src, P = g["capacity"], g["max_prompt_len"], g["prompt_tokens"]
    rng = np.random.default_rng(32)
    H, D = 1, 4
    src, dst = _prefill_generate(rng, 1, H, D, S_src, S_dst, [P])
    (K, V), mask = oracle.copy_kvcache(src, dst, [P], np.zeros((1, S_dst), dtype=np.int32))
    printed = {p["generated_token"]: p["valid_rows"] for p in g["points"]}
    for n in range(2, 12):
        K, V, mask = oracle.kv_append(K, V, random_bf16(rng, (1, H, D)),
                                      random_bf16(rng, (1, H, D)), [int(mask.sum())], mask)
        if n in printed:
            assert int(mask.sum()) == printed[n]
        assert int(mask.sum()) == n + 3


def test_trim_equals_attention_over_the_kept_rows():
    rng = np.random.default_rng(33)
    B, H, D, S = 2, 2, 8, 40
    K = random_bf16(rng, (B, H, S, D))
    V = random_bf16(rng, (B, H, S, D))
    mask = np.zeros((B, S), dtype=np.int32)
    mask[0, :30] = 1
    mask[1, :12] = 1
    trimmed = oracle.trim_kvcache(mask, [25, 12])
    q = rng.standard_normal((B, H, D))
    got, _ = oracle.decode_static(q, K, V, mask=trimmed)
    want, _ = oracle.decode_static(q, K, V, valid_len=[25, 12])
    assert np.array_equal(got, want)
    empty = oracle.trim_kvcache(mask, [0, 0])
    out, lse = oracle.decode_static(q, K, V, mask=empty)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_copy_and_trim_reject_lengths_outside_the_buffers():
    rng = np.random.default_rng(34)
    src, dst = _prefill_generate(rng, 1, 1, 8, 16, 20, [16])
    with pytest.raises(ValueError):
        oracle.copy_kvcache(src, dst, [17])
    with pytest.raises(ValueError):
        oracle.copy_kvcache(src, dst, [-1])
    with pytest.raises(ValueError):
        oracle.trim_kvcache(np.ones((1, 20), dtype=np.int32), [21])
