"""GPU parity: the sparse kernel over an FP4 latent cache -- the quantising latent
append (codes and scales bit-exact) and sparse top-k attention over E2M1 codes, two
per byte, with row scales (within the attention tolerance) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy
from oracle import round_to_bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_dev(bits_u16):
    return torch.from_numpy(bits_u16.view(np.int16)).to(DEV).view(torch.bfloat16)


def run(case, **kw):
    out, lse = dakv.sparse_topk_attn_fp4(case.q, case.codes, case.scale, case.indices,
                                         d_v=case.d_v, sm_scale=case.sm_scale, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


def ref(case, seqs=None):
    q, codes, scale, idx = bits(case.q), case.codes, case.scale, npy(case.indices)
    if seqs is not None:
        q, idx, codes, scale = q[seqs], idx[seqs], codes[seqs], scale[seqs]
    return oracle.sparse_topk_attn_fp4(q, npy(codes), npy(scale).astype(np.float64), idx,
                                       case.d_v, case.sm_scale)


def test_latent_append_fp4_codes_and_scales_bit_exact():
    rng = np.random.default_rng(121)
    B, s_kv, d = 5, 9, 576
    mag = np.exp(rng.uniform(-60, 60, size=(B, 1)))
    rows = round_to_bf16_bits(rng.standard_normal((B, d)) * mag)
    rows[1, :] = 0                                   # a zero row: scale 1, +0 codes
    codes0 = rng.integers(0, 256, size=(B, s_kv, d // 2)).astype(np.uint8)
    scale0 = np.exp2(rng.integers(-8, 0, size=(B, s_kv))).astype(np.float32)
    pos = np.array([0, 8, 3, 4, 9], dtype=np.int32)  # the last one is outside
    codes = torch.from_numpy(codes0.copy()).to(DEV)
    scale = torch.from_numpy(scale0.copy()).to(DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.latent_append_fp4(codes, scale, bf16_dev(rows), torch.from_numpy(pos).to(DEV),
                           err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_WRITE_POS
    r_codes, r_scale = oracle.latent_append_fp4(codes0[:4], scale0[:4].astype(np.float64),
                                                rows[:4], pos[:4])
    assert np.array_equal(npy(codes)[:4], r_codes)
    assert np.array_equal(npy(scale)[:4].astype(np.float64), r_scale)
    assert np.array_equal(npy(codes)[4], codes0[4]) and np.array_equal(npy(scale)[4], scale0[4])


@pytest.mark.parametrize("B,s_q,Hq,s_kv,topk", [
    (2, 1, 16, 1000, 300),     # two index splits, ragged last tile
    (1, 2, 48, 700, 65),       # two tokens, a head group with an idle head block
    (2, 1, 64, 5000, 512),     # one whole split
    (2, 1, 128, 4096, 2048),   # the config's heads and top-k at a smaller context
    (3, 2, 32, 64, 1),         # a single index per token
    (2, 1, 16, 100, 0),        # no index: zero output, lse -inf
])
def test_sparse_fp4_matches_oracle(B, s_q, Hq, s_kv, topk):
    print(f"sparse fp4 B={B} s_q={s_q} Hq={Hq} s_kv={s_kv} topk={topk}", flush=True)
    case = workloads.sparse_fp4_case(B, s_q, Hq, s_kv, topk, device=DEV, seed=150 + topk)
    out, lse = run(case)
    r_out, r_lse = ref(case)
    assert_attention_close(out, r_out)
    assert_lse_close(lse, r_lse)


def test_sparse_fp4_equals_bf16_kernel_over_the_dequantised_rows():
    """The FP4 tile holds code value times scale in bf16, exactly the numbers a bf16
    cache of the dequantised rows holds, and the rest of the pass is shared: the two
    calls agree bit for bit."""
    case = workloads.sparse_fp4_case(2, 2, 32, 3000, 1000, device=DEV, seed=160)
    deq = oracle.fp4.dequantize(npy(case.codes), npy(case.scale).astype(np.float64))
    kv_bits = round_to_bf16_bits(deq)
    assert np.array_equal(oracle.widen(kv_bits), deq)
    o8, l8 = run(case)
    ob, lb = dakv.sparse_topk_attn(case.q, bf16_dev(kv_bits), case.indices, d_v=case.d_v,
                                   sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(o8, npy(ob)) and np.array_equal(l8, npy(lb))


def test_sparse_fp4_out_of_range_index_is_flagged_and_skipped():
    case = workloads.sparse_fp4_case(1, 1, 16, 200, 40, device=DEV, seed=161)
    idx = npy(case.indices).copy()
    good = idx.copy()
    idx[0, 0, 7] = 200
    idx[0, 0, 30] = -5
    case.indices = torch.from_numpy(idx).to(DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _ = run(case, err_flag=flag)
    assert int(flag.item()) & dakv._lib.ERR_SPARSE_INDEX
    keep = [i for i in range(40) if i not in (7, 30)]
    r_out, _ = oracle.sparse_topk_attn_fp4(bits(case.q), npy(case.codes),
                                           npy(case.scale).astype(np.float64),
                                           good[:, :, keep], case.d_v, case.sm_scale)
    assert_attention_close(out, r_out)


def test_sparse_fp4_full_size_every_sequence():
    """Batch 16, 128 heads, d_qk 576 / d_v 512, context 32768, top-2048 over an FP4
    latent cache: every output of every sequence against the oracle."""
    print("sparse fp4 full size", flush=True)
    case = workloads.sparse_fp4_case(16, 1, 128, 32768, 2048, device=DEV, seed=162)
    out, lse = run(case)
    for b in range(16):
        r_out, r_lse = ref(case, seqs=slice(b, b + 1))
        assert_attention_close(out[b:b + 1], r_out)
        assert_lse_close(lse[b:b + 1], r_lse)
