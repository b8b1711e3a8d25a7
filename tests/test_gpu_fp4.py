"""GPU parity: the FP4 (E2M1) KV cache -- quantising append (codes and scales bit-exact)
and decode attention over E2M1 codes (within the attention tolerance) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, npy
from oracle import fp4, round_to_bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_dev(bits_u16):
    return torch.from_numpy(bits_u16.view(np.int16)).to(DEV).view(torch.bfloat16)


def random_scales(rng, shape):
    """Row scales 2^-3 .. 2^0: those of quantised rows with max |x| up to 6 (O(1) rows)."""
    return np.exp2(rng.integers(-3, 1, size=shape)).astype(np.float32)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_append_fp4_codes_and_scales_bit_exact(D):
    rng = np.random.default_rng(300 + D)
    B, H, cap = 3, 4, 10
    mag = np.exp(rng.uniform(-40, 40, size=(B, H, 1)))
    k = rng.standard_normal((B, H, D)) * mag
    v = rng.standard_normal((B, H, D))
    k[0, 0] = 0.0
    v[1, 2, :] = -0.0
    # every E2M1 midpoint at scale 2^-1, plus the largest value fixing that scale
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    v[2, 1, :] = np.resize(np.concatenate([mids, -mids]), D) * 0.5
    v[2, 1, 0] = 6.0 * 0.5
    k_bits, v_bits = round_to_bf16_bits(k), round_to_bf16_bits(v)
    kc = np.zeros((B, H, cap, D // 2), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.ones((B, H, cap), np.float32)
    vs = np.ones_like(ks)
    pos = [0, 4, cap - 1]
    mask = np.zeros((B, cap), np.int32)
    want = oracle.kv_append_fp4(kc, vc, ks, vs, k_bits, v_bits, pos, mask)
    t = [torch.from_numpy(a).to(DEV) for a in (kc, vc, ks, vs)]
    m = torch.from_numpy(mask).to(DEV)
    dakv.kv_append_fp4(*t, bf16_dev(k_bits), bf16_dev(v_bits),
                       torch.tensor(pos, dtype=torch.int32, device=DEV), mask=m)
    torch.cuda.synchronize()
    assert np.array_equal(npy(t[0]), want[0])
    assert np.array_equal(npy(t[1]), want[1])
    assert np.array_equal(npy(t[2]).astype(np.float64), want[2])
    assert np.array_equal(npy(t[3]).astype(np.float64), want[3])
    assert np.array_equal(npy(m), want[4])


def run_fp4(q, kc, vc, ks, vs, mask, valid_len, **kw):
    dev = [torch.from_numpy(a).to(DEV) for a in (q, kc, vc, ks, vs)]
    m = None if mask is None else torch.from_numpy(mask).to(DEV)
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32, device=DEV)
    out, lse = dakv.decode_attn_static_fp4(*dev, mask=m, valid_len=vl, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


@pytest.mark.parametrize("D,cap,lengths", [(64, 1152, [4, 5, 103, 1152]),
                                           (128, 700, [1, 63, 64, 65, 700]),
                                           (128, 4096, [4096, 1999])])
def test_decode_fp4_matches_oracle(D, cap, lengths):
    rng = np.random.default_rng(310 + D + cap)
    B, H = len(lengths), 3
    kc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    mask = (rng.uniform(size=(B, cap)) < 0.8).astype(np.int32)
    q = (rng.standard_normal((B, H, D)) * 0.1).astype(np.float32)
    out, lse = run_fp4(q, kc, vc, ks, vs, mask, lengths)
    ref_out, ref_lse = oracle.decode_static_fp4(q, kc, vc, ks, vs, mask=mask, valid_len=lengths)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
    one, _ = run_fp4(q, kc, vc, ks, vs, mask, lengths, num_splits=1)
    assert_attention_close(one, ref_out)


def test_quantise_on_device_then_attend_full_size_sampled():
    """LLaMA-7B-shaped layer, batch 8, capacity 4096, FP4 cache: a new row quantised by
    the device append, then decode attention; sampled sequences vs the oracle."""
    print("fp4 full size", flush=True)
    rng = np.random.default_rng(320)
    B, H, cap, D = 8, 32, 4096, 128
    lengths = [3431, 1072, 448, 1223, 1695, 3336, 1849, 377]
    kc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    t = [torch.from_numpy(a).to(DEV) for a in (kc, vc, ks, vs)]
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    pos = [L - 1 for L in lengths]
    dakv.kv_append_fp4(*t, bf16_dev(k_new), bf16_dev(v_new),
                       torch.tensor(pos, dtype=torch.int32, device=DEV))
    q = (rng.standard_normal((B, H, D)) * 0.1).astype(np.float32)
    out, lse = dakv.decode_attn_static_fp4(torch.from_numpy(q).to(DEV), *t,
                                           valid_len=torch.tensor(lengths, dtype=torch.int32,
                                                                  device=DEV))
    torch.cuda.synchronize()
    out, lse = npy(out), npy(lse)
    for b in (0, 3, 7):
        sel = slice(b, b + 1)
        codes = [npy(x[sel]) for x in t]
        ref_out, ref_lse = oracle.decode_static_fp4(q[sel], *codes, valid_len=[lengths[b]])
        assert_attention_close(out[sel], ref_out)
        assert_lse_close(lse[sel], ref_lse)
        kq, kscale = fp4.quantize_rows(k_new[b])
        assert np.array_equal(codes[0][0, :, pos[b]], kq)
        assert np.array_equal(codes[2][0, :, pos[b]].astype(np.float64), kscale)


# ------------------------------------------------ fused append + attend (FP4 cache)


def run_step_fp4(q, kc, vc, ks, vs, k_new, v_new, pos, mask, valid_len, **kw):
    dev = [torch.from_numpy(a).to(DEV) for a in (q, kc, vc, ks, vs)]
    m = None if mask is None else torch.from_numpy(mask).to(DEV)
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32, device=DEV)
    out, lse = dakv.decode_step_static_fp4(
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
def test_decode_step_fp4_matches_append_then_attend(D, cap, lengths, pos, use_mask, use_len):
    """Fused append + attend over the FP4 cache: the stored codes, scales and mask are
    bit-exact with the oracle's kv_append_fp4, the output matches decode_static_fp4 on
    that state (a position at or past the valid length is stored but not attended)."""
    rng = np.random.default_rng(71 + D + cap)
    B, H = len(lengths), 3
    kc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    mask = (rng.uniform(size=(B, cap)) < 0.8).astype(np.int32) if use_mask else None
    if mask is not None:
        mask[np.arange(B), pos] = 0          # the append must set it
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)) * 3.0)
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)) * 0.5)
    q = (rng.standard_normal((B, H, D)) * 0.2).astype(np.float32)
    vl = lengths if use_len else None
    out, lse, state = run_step_fp4(q, kc, vc, ks, vs, k_new, v_new, pos, mask, vl)
    want = oracle.kv_append_fp4(kc, vc, ks, vs, k_new, v_new, pos, mask)
    assert np.array_equal(state[0], want[0]) and np.array_equal(state[1], want[1])
    assert np.array_equal(state[2].astype(np.float64), want[2])
    assert np.array_equal(state[3].astype(np.float64), want[3])
    if mask is not None:
        assert np.array_equal(state[4], want[4])
    ref_out, ref_lse = oracle.decode_static_fp4(q, *want[:4], mask=want[4], valid_len=vl)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_decode_step_fp4_equals_the_two_calls_and_flags_bad_position():
    rng = np.random.default_rng(81)
    B, H, cap, D = 3, 4, 2048, 128
    lengths, pos = [2048, 1000, 77], [1500, 999, 5000]
    kc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(B, H, cap, D // 2)).astype(np.uint8)
    ks, vs = random_scales(rng, (B, H, cap)), random_scales(rng, (B, H, cap))
    k_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    v_new = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    q = (rng.standard_normal((B, H, D)) * 0.2).astype(np.float32)
    vl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    wp = torch.tensor(pos, dtype=torch.int32, device=DEV)
    for splits in (0, 1, 13):
        a = [torch.from_numpy(x).to(DEV) for x in (kc, vc, ks, vs)]
        b = [x.clone() for x in a]
        qd = torch.from_numpy(q).to(DEV)
        fa = torch.zeros(1, dtype=torch.int32, device=DEV)
        fb = torch.zeros(1, dtype=torch.int32, device=DEV)
        o1, l1 = dakv.decode_step_static_fp4(qd, *a, bf16_dev(k_new), bf16_dev(v_new), wp,
                                             valid_len=vl, num_splits=splits, err_flag=fa)
        dakv.kv_append_fp4(*b, bf16_dev(k_new), bf16_dev(v_new), wp, err_flag=fb)
        o2, l2 = dakv.decode_attn_static_fp4(qd, *b, valid_len=vl, num_splits=splits)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert int(fa.item()) & dakv._lib.ERR_WRITE_POS
        assert int(fb.item()) & dakv._lib.ERR_WRITE_POS
