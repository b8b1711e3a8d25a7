"""The skip-scale branch of the sparse kernel, targeted (FlashMLA on Huawei Ascend,
"Course of computation": the running max used for the exponentials is only moved
when a block of the index list raises it by more than 6 nats; "How to synchronise
skip-scale?": every core that shares the head takes the same decision).

The kernel walks each 512-index split in 64-row tiles.  The inputs here are built
so that, in every split, a later tile raises every head's running max by just
under 6 nats (the branch is not taken: exponentials up to e^5.9 enter the sums
unscaled) or by just over 6 nats (taken: the accumulators are rescaled), and a
third case where five rows spread over the four splits dominate a top-2048 list
by about 12 nats.  Each runs over bf16, FP8 and FP4 latent caches.

Design: query head h (of 128) is c times the unit vector on dimension h plus
noise of size 0.003 on dimensions 128..575; the latent rows hold values below 2
on dimensions 0..127, except one row in tile 0 of the split holding 4 there and
one row in a later tile holding 12, so the jump is sm_scale * c * 8 up to the
noise; c is picked in bf16 for 5.9 or 6.1 nats.  4 and 12 are exact in bf16, in
E4M3 with scale 1 and in E2M1 (6 with scale 2).  test_designed_jumps_straddle_
the_threshold checks, from the dequantised inputs, that every (sequence, split,
head) sees the intended jump.
"""

import numpy as np
import pytest
import torch

import oracle
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, npy

DEV = "cuda:0"
D_QK, D_V, HQ = 576, 512, 128
SM = 1.0 / 24.0                      # 1 / sqrt(576)
SPLIT, TILE = 512, 64
B, S_KV, TOPK = 2, 4096, 2048
V_LOW, V_HIGH = 4.0, 12.0
DOMINANT = [17, 600, 1100, 1101, 2040]   # positions in the index list
CASES = {"under": 5.9, "over": 6.1, "dominant": None}


def to_bf16_bits(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def e4m3_bytes(rng, shape, emax):
    """Finite E4M3 codes with exponent field 1..emax (|value| < 2^(emax - 6))."""
    s = rng.integers(0, 2, shape)
    e = rng.integers(1, emax + 1, shape)
    m = rng.integers(0, 8, shape)
    return (s << 7 | e << 3 | m).astype(np.uint8)


def e2m1_nibbles(rng, shape, cmax):
    """E2M1 codes with magnitude code 0..cmax (value <= {0,.5,1,1.5,2,3,4,6}[cmax])."""
    return (rng.integers(0, 2, shape) << 3 | rng.integers(0, cmax + 1, shape)).astype(np.uint8)


def design(fmt, kind, seed):
    """Inputs for one case.  Returns a dict with the query bits, the latent cache in
    the format's stored form, the index list and the designated positions."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(S_KV, TOPK, replace=False) for _ in range(B)]).astype(np.int32)
    if kind == "dominant":
        high_pos = [list(DOMINANT) for _ in range(B)]
        low_pos = [[] for _ in range(B)]
        c = 12.0 / (SM * (V_HIGH - 2.0))
    else:
        low_pos, high_pos = [], []
        for _ in range(B):
            lo, hi = [], []
            for k in range(TOPK // SPLIT):
                lo.append(SPLIT * k + int(rng.integers(0, TILE)))
                hi.append(SPLIT * k + TILE * (k + 1) + int(rng.integers(0, TILE)))
            low_pos.append(lo)
            high_pos.append(hi)
        c = CASES[kind] / (SM * (V_HIGH - V_LOW))
    c = float(bf16_value(to_bf16_bits([c]))[0])
    q = np.zeros((B, HQ, D_QK))
    q[:, np.arange(HQ), np.arange(HQ)] = c
    q[:, :, 128:] = 0.003 * rng.standard_normal((B, HQ, D_QK - 128))
    case = {"q": to_bf16_bits(q), "idx": idx, "low": low_pos, "high": high_pos, "c": c}
    if fmt == "bf16":
        val = np.empty((B, S_KV, D_QK))
        val[:, :, :128] = rng.uniform(-1.9, 1.9, (B, S_KV, 128))
        val[:, :, 128:] = rng.standard_normal((B, S_KV, D_QK - 128))
        for b in range(B):
            val[b, idx[b, low_pos[b]], :128] = V_LOW
            val[b, idx[b, high_pos[b]], :128] = V_HIGH
        case["kv"] = to_bf16_bits(val)
    elif fmt == "fp8":
        codes = np.empty((B, S_KV, D_QK), np.uint8)
        codes[:, :, :128] = e4m3_bytes(rng, (B, S_KV, 128), 7)
        codes[:, :, 128:] = e4m3_bytes(rng, (B, S_KV, D_QK - 128), 8)
        for b in range(B):
            codes[b, idx[b, low_pos[b]], :128] = 0x48     # 4 = 2^2
            codes[b, idx[b, high_pos[b]], :128] = 0x54    # 12 = 1.5 * 2^3
        case["codes"], case["scale"] = codes, np.ones((B, S_KV), np.float32)
    else:
        nib = np.empty((B, S_KV, D_QK), np.uint8)
        nib[:, :, :128] = e2m1_nibbles(rng, (B, S_KV, 128), 4)
        nib[:, :, 128:] = e2m1_nibbles(rng, (B, S_KV, D_QK - 128), 7)
        scale = np.ones((B, S_KV), np.float32)
        for b in range(B):
            nib[b, idx[b, low_pos[b]], :128] = 6             # 4, scale 1
            rows = idx[b, high_pos[b]]
            nib[b, rows, :128] = 7                           # 6, scale 2 -> 12
            nib[b, rows, 128:] = e2m1_nibbles(rng, (len(rows), D_QK - 128), 4)
            scale[b, rows] = 2.0
        case["codes"] = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
        case["scale"] = scale
    return case


def dequantised(fmt, case):
    if fmt == "bf16":
        return bf16_value(case["kv"])
    if fmt == "fp8":
        return oracle.e4m3_decode(case["codes"]) * case["scale"][..., None].astype(np.float64)
    return oracle.fp4.dequantize(case["codes"], case["scale"])


SEEDS = {("bf16", "under"): 301, ("bf16", "over"): 302, ("bf16", "dominant"): 303,
         ("fp8", "under"): 311, ("fp8", "over"): 312, ("fp8", "dominant"): 313,
         ("fp4", "under"): 321, ("fp4", "over"): 322, ("fp4", "dominant"): 323}


@pytest.mark.parametrize("fmt,kind", sorted(SEEDS))
def test_designed_jumps_straddle_the_threshold(fmt, kind):
    """The inputs do what the GPU cases rely on (checked on the CPU, in fp64)."""
    case = design(fmt, kind, SEEDS[(fmt, kind)])
    val = dequantised(fmt, case)
    q = bf16_value(case["q"])
    for b in range(B):
        s = SM * (val[b, case["idx"][b]] @ q[b].T)          # [topk, heads], nats
        if kind == "dominant":
            top = s[DOMINANT]
            rest = np.delete(s, DOMINANT, axis=0)
            assert np.all(top.min(axis=0) - rest.max(axis=0) > 11.5)
            continue
        for k in range(TOPK // SPLIT):
            blk = s[SPLIT * k:SPLIT * (k + 1)]
            tiles = blk.reshape(SPLIT // TILE, TILE, HQ).max(axis=1)   # [tiles, heads]
            t_hi = (case["high"][b][k] - SPLIT * k) // TILE
            before = tiles[:t_hi].max(axis=0)
            jump = tiles[t_hi] - before
            if kind == "under":
                assert np.all((jump > 5.75) & (jump < 5.99)), (b, k, jump.min(), jump.max())
            else:
                assert np.all((jump > 6.01) & (jump < 6.25)), (b, k, jump.min(), jump.max())
            # tile 0 holds the split's earlier maximum; no other tile moves it by > 1
            assert np.all(tiles[1:t_hi].max(axis=0, initial=-np.inf) <= tiles[0] + 1.0)
            assert np.all(tiles[t_hi + 1:] <= tiles[t_hi][None] + 1.0)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt,kind", sorted(SEEDS))
def test_skip_scale_branch_matches_oracle(fmt, kind):
    print(f"sparse skip-scale {fmt} {kind}", flush=True)
    case = design(fmt, kind, SEEDS[(fmt, kind)])
    q = torch.from_numpy(case["q"].view(np.int16)).to(DEV).view(torch.bfloat16)
    idx = torch.from_numpy(case["idx"]).to(DEV)
    if fmt == "bf16":
        kv = torch.from_numpy(case["kv"].view(np.int16)).to(DEV).view(torch.bfloat16)
        out, lse = dakv.sparse_topk_decode_attn(q, kv, idx, d_v=D_V, sm_scale=SM)
        torch.cuda.synchronize()
        r_out, r_lse = oracle.sparse_topk_decode(case["q"], case["kv"], case["idx"], D_V, SM)
    else:
        codes = torch.from_numpy(case["codes"]).to(DEV)
        scale = torch.from_numpy(case["scale"]).to(DEV)
        fn = dakv.sparse_topk_attn_fp8 if fmt == "fp8" else dakv.sparse_topk_attn_fp4
        ref = oracle.sparse_topk_attn_fp8 if fmt == "fp8" else oracle.sparse_topk_attn_fp4
        out, lse = fn(q[:, None].contiguous(), codes, scale, idx[:, None].contiguous(), d_v=D_V,
                      sm_scale=SM)
        torch.cuda.synchronize()
        r_out, r_lse = ref(case["q"][:, None], case["codes"], case["scale"].astype(np.float64),
                           case["idx"][:, None], D_V, SM)
        out, lse = out[:, 0], lse[:, 0]
        r_out, r_lse = r_out[:, 0], r_lse[:, 0]
    assert_attention_close(npy(out), r_out)
    assert_lse_close(npy(lse), r_lse)
