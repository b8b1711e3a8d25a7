"""GPU parity: the FP8 KV cache -- quantising append (codes and scales bit-exact)
and decode attention over E4M3 codes (within the attention tolerance) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy
from oracle import round_to_bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_dev(bits_u16):
    return torch.from_numpy(bits_u16.view(np.int16)).to(DEV).view(torch.bfloat16)


def random_codes(rng, shape):
    """Finite E4M3 codes (every byte but the two NaN codes)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = 0x7E
    return c


def random_scales(rng, shape):
    """Row scales 2^-12 .. 2^-6: those of quantised rows with max |x| up to 7, as the
    O(1) K and V rows of the attention workloads give (codes reach 448 * 2^-6)."""
    return np.exp2(rng.integers(-12, -5, size=shape)).astype(np.float32)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_append_fp8_codes_and_scales_bit_exact(D):
    rng = np.random.default_rng(100 + D)
    B, H, cap = 3, 5, 12
    mag = np.exp(rng.uniform(-60, 60, size=(B, H, 1)))
    k = rng.standard_normal((B, H, D)) * mag
    v = rng.standard_normal((B, H, D))
    k[0, 0] = 0.0                                    # a zero row
    v[1, 2, :] = -0.0                                # negative zeros
    # exact ties of the E4M3 grid at a chosen scale
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    v[2, 1, :] = np.resize(mids[-D:], D) * 2.0 ** -3
    v[2, 1, 0] = 448.0 * 2.0 ** -3                   # makes the row's scale 2^-3
    k_bits, v_bits = round_to_bf16_bits(k), round_to_bf16_bits(v)
    kc = np.zeros((B, H, cap, D), np.uint8)
    vc = np.zeros((B, H, cap, D), np.uint8)
    ks = np.ones((B, H, cap), np.float32)
    vs = np.ones((B, H, cap), np.float32)
    pos = [0, 5, cap - 1]
    mask = np.zeros((B, cap), np.int32)
    want = oracle.kv_append_fp8(kc, vc, ks, vs, k_bits, v_bits, pos, mask)
    t = [torch.from_numpy(a).to(DEV) for a in (kc, vc, ks, vs)]
    m = torch.from_numpy(mask).to(DEV)
    dakv.kv_append_fp8(*t, bf16_dev(k_bits), bf16_dev(v_bits),
                       torch.tensor(pos, dtype=torch.int32, device=DEV), mask=m)
    torch.cuda.synchronize()
    assert np.array_equal(npy(t[0]), want[0])
    assert np.array_equal(npy(t[1]), want[1])
    assert np.array_equal(npy(t[2]).astype(np.float64), want[2])
    assert np.array_equal(npy(t[3]).astype(np.float64), want[3])
    assert np.array_equal(npy(m), want[4])


def test_append_fp8_position_outside_is_flagged_and_skipped():
    B, H, cap, D = 2, 2, 8, 64
    t = [torch.zeros((B, H, cap, D), dtype=torch.uint8, device=DEV) for _ in range(2)]
    s = [torch.ones((B, H, cap), dtype=torch.float32, device=DEV) for _ in range(2)]
    new = torch.ones((B, H, D), dtype=torch.bfloat16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.kv_append_fp8(t[0], t[1], s[0], s[1], new, new,
                       torch.tensor([8, 3], dtype=torch.int32, device=DEV), err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_WRITE_POS
    assert int(t[0][0].count_nonzero()) == 0 and int(t[0][1, :, 3].count_nonzero()) > 0


def run_fp8(q, kc, vc, ks, vs, mask, valid_len, **kw):
    dev = [torch.from_numpy(a).to(DEV) for a in (q, kc, vc, ks, vs)]
    m = None if mask is None else torch.from_numpy(mask).to(DEV)
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32, device=DEV)
    out, lse = dakv.decode_attn_static_fp8(*dev, mask=m, valid_len=vl, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


@pytest.mark.parametrize("D,cap,lengths", [(64, 1152, [4, 5, 103, 1152]),
                                           (128, 700, [1, 63, 64, 65, 700]),
                                           (128, 4096, [4096, 1999])])
def test_decode_fp8_matches_oracle(D, cap, lengths):
    rng = np.random.default_rng(7 + D + cap)
    B, H = len(lengths), 3
    kc, vc = random_codes(rng, (B, H, cap, D)), random_codes(rng, (B, H, cap, D))
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    mask = (rng.uniform(size=(B, cap)) < 0.8).astype(np.int32)
    q = (rng.standard_normal((B, H, D)) * 0.05).astype(np.float32)
    out, lse = run_fp8(q, kc, vc, ks, vs, mask, lengths)
    ref_out, ref_lse = oracle.decode_static_fp8(q, kc, vc, ks, vs, mask=mask, valid_len=lengths)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_decode_fp8_split_counts_agree_and_empty_sequence():
    rng = np.random.default_rng(9)
    B, H, cap, D = 2, 2, 3000, 128
    kc, vc = random_codes(rng, (B, H, cap, D)), random_codes(rng, (B, H, cap, D))
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    q = (rng.standard_normal((B, H, D)) * 0.05).astype(np.float32)
    a, _ = run_fp8(q, kc, vc, ks, vs, None, [2999, 0])
    one, lse1 = run_fp8(q, kc, vc, ks, vs, None, [2999, 0], num_splits=1)
    many, _ = run_fp8(q, kc, vc, ks, vs, None, [2999, 0], num_splits=40)
    assert np.max(np.abs(a - one)) <= 1e-5 * np.max(np.abs(one))
    assert np.max(np.abs(many - one)) <= 1e-5 * np.max(np.abs(one))
    assert np.all(a[1] == 0) and np.all(np.isneginf(lse1[1]))


def test_quantise_on_device_then_attend_full_size_sampled():
    """LLaMA-7B-shaped layer, batch 8, capacity 4096, FP8 cache: rows quantised by
    the device append, then decode attention; sampled sequences vs the oracle."""
    print("fp8 full size", flush=True)
    rng = np.random.default_rng(11)
    B, H, cap, D = 8, 32, 4096, 128
    lengths = [3431, 1072, 448, 1223, 1695, 3336, 1849, 377]
    kc, vc = random_codes(rng, (B, H, cap, D)), random_codes(rng, (B, H, cap, D))
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    t = [torch.from_numpy(a).to(DEV) for a in (kc, vc, ks, vs)]
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    pos = [L - 1 for L in lengths]
    dakv.kv_append_fp8(*t, bf16_dev(k_new), bf16_dev(v_new),
                       torch.tensor(pos, dtype=torch.int32, device=DEV))
    q = (rng.standard_normal((B, H, D)) * 0.05).astype(np.float32)
    qd = torch.from_numpy(q).to(DEV)
    out, lse = dakv.decode_attn_static_fp8(qd, *t, valid_len=torch.tensor(lengths, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    out, lse = npy(out), npy(lse)
    for b in (0, 2, 7):
        sel = slice(b, b + 1)
        codes = [npy(x[sel]) for x in t]
        ref_out, ref_lse = oracle.decode_static_fp8(q[sel], *codes, valid_len=[lengths[b]])
        assert_attention_close(out[sel], ref_out)
        assert_lse_close(lse[sel], ref_lse)
        # the appended row is the oracle's quantisation of the new token
        kq, kscale = oracle.quantize_rows(k_new[b])
        assert np.array_equal(codes[0][0, :, pos[b]], kq)
        assert np.array_equal(codes[2][0, :, pos[b]].astype(np.float64), kscale)


def run_step_fp8(q, kc, vc, ks, vs, k_new, v_new, pos, mask, valid_len, **kw):
    dev = [torch.from_numpy(a).to(DEV) for a in (q, kc, vc, ks, vs)]
    m = None if mask is None else torch.from_numpy(mask).to(DEV)
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32, device=DEV)
    out, lse = dakv.decode_step_static_fp8(
        *dev, bf16_dev(k_new), bf16_dev(v_new), torch.tensor(pos, dtype=torch.int32, device=DEV),
        mask=m, valid_len=vl, **kw)
    torch.cuda.synchronize()
    state = [npy(x) for x in dev[1:]] + [None if m is None else npy(m)]
    return npy(out), npy(lse), state


@pytest.mark.parametrize("D,cap,lengths,pos,use_mask,use_len", [
    (64, 1152, [5, 103, 1152, 640], [4, 102, 1151, 700], True, True),
    (128, 700, [1, 64, 65, 700, 300], [0, 63, 64, 699, 500], True, True),
    (128, 4096, [4096, 1999], [4000, 1998], False, True),
    (128, 300, [300, 300], [0, 257], True, False),
])
def test_decode_step_fp8_matches_append_then_attend(D, cap, lengths, pos, use_mask, use_len):
    """Fused append + attend: the stored codes, scales and mask are bit-exact with the
    oracle's kv_append_fp8, the output matches decode_static_fp8 on that state (a
    position at or past the valid length is stored but not attended)."""
    rng = np.random.default_rng(31 + D + cap)
    B, H = len(lengths), 3
    kc, vc = random_codes(rng, (B, H, cap, D)), random_codes(rng, (B, H, cap, D))
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    mask = (rng.uniform(size=(B, cap)) < 0.8).astype(np.int32) if use_mask else None
    if mask is not None:
        mask[np.arange(B), pos] = 0          # the append must set it
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)) * 3.0)
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)) * 0.01)
    q = (rng.standard_normal((B, H, D)) * 0.05).astype(np.float32)
    vl = lengths if use_len else None
    out, lse, state = run_step_fp8(q, kc, vc, ks, vs, k_new, v_new, pos, mask, vl)
    want = oracle.kv_append_fp8(kc, vc, ks, vs, k_new, v_new, pos, mask)
    assert np.array_equal(state[0], want[0]) and np.array_equal(state[1], want[1])
    assert np.array_equal(state[2].astype(np.float64), want[2])
    assert np.array_equal(state[3].astype(np.float64), want[3])
    if mask is not None:
        assert np.array_equal(state[4], want[4])
    ref_out, ref_lse = oracle.decode_static_fp8(q, *want[:4], mask=want[4], valid_len=vl)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_decode_step_fp8_equals_the_two_calls_and_flags_bad_position():
    rng = np.random.default_rng(41)
    B, H, cap, D = 3, 4, 2048, 128
    lengths, pos = [2048, 1000, 77], [1500, 999, 5000]
    kc, vc = random_codes(rng, (B, H, cap, D)), random_codes(rng, (B, H, cap, D))
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    q = (rng.standard_normal((B, H, D)) * 0.05).astype(np.float32)
    vl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    wp = torch.tensor(pos, dtype=torch.int32, device=DEV)
    for splits in (0, 1, 13):
        a = [torch.from_numpy(x).to(DEV) for x in (kc, vc, ks, vs)]
        b = [x.clone() for x in a]
        qd = torch.from_numpy(q).to(DEV)
        fa = torch.zeros(1, dtype=torch.int32, device=DEV)
        fb = torch.zeros(1, dtype=torch.int32, device=DEV)
        o1, l1 = dakv.decode_step_static_fp8(qd, *a, bf16_dev(k_new), bf16_dev(v_new), wp,
                                             valid_len=vl, num_splits=splits, err_flag=fa)
        dakv.kv_append_fp8(*b, bf16_dev(k_new), bf16_dev(v_new), wp, err_flag=fb)
        o2, l2 = dakv.decode_attn_static_fp8(qd, *b, valid_len=vl, num_splits=splits)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert int(fa.item()) & dakv._lib.ERR_WRITE_POS
        assert int(fb.item()) & dakv._lib.ERR_WRITE_POS
