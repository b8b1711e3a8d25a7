"""GPU parity: sparse_topk_decode_attn (MFMA) vs the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(case, **kw):
    out, lse = dakv.sparse_topk_decode_attn(case.q, case.kv, case.indices, d_v=case.d_v,
                                            sm_scale=case.sm_scale, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


def ref(case, rows=None):
    q, kv, idx = bits(case.q), case.kv, npy(case.indices)
    if rows is not None:
        q, idx = q[rows], idx[rows]
        kv = case.kv[rows]
    return oracle.sparse_topk_decode(q, bits(kv), idx, case.d_v, case.sm_scale)


@pytest.mark.parametrize("B,Hq,s_kv,topk", [
    (2, 16, 1000, 300),     # two splits, ragged last tile
    (1, 48, 700, 33),       # one head group with an idle wave, ragged tile
    (2, 64, 5000, 512),
    (2, 128, 4096, 2048),   # the config's heads and top-k at a smaller context
    (3, 32, 64, 1),         # a single index
    (2, 32, 3000, 1000),    # two index splits, the second ragged
    (2, 16, 100, 0),        # no index: zero output, lse -inf
    (1, 16, 8000, 5000),    # ten index splits: the merge takes them in two batches
])
def test_sparse_matches_oracle(B, Hq, s_kv, topk):
    print(f"sparse B={B} Hq={Hq} s_kv={s_kv} topk={topk}", flush=True)
    case = workloads.sparse_case(B, Hq, s_kv, topk, device=DEV, seed=80 + topk)
    out, lse = run(case)
    r_out, r_lse = ref(case)
    assert_attention_close(out, r_out)
    assert_lse_close(lse, r_lse)


def test_sparse_full_index_is_dense_attention():
    B, Hq, s_kv = 1, 32, 640
    case = workloads.sparse_case(B, Hq, s_kv, s_kv, device=DEV, seed=90)
    case.indices = torch.arange(s_kv, dtype=torch.int32, device=DEV)[None].repeat(B, 1).contiguous()
    out, _ = run(case)
    r_out, _ = ref(case)
    assert_attention_close(out, r_out)


def test_sparse_duplicates_count_twice_and_order_is_irrelevant():
    case = workloads.sparse_case(2, 32, 300, 100, device=DEV, seed=91)
    idx = npy(case.indices).copy()
    idx[:, 50:60] = idx[:, 0:10]                      # duplicates
    case.indices = torch.from_numpy(idx).to(DEV)
    out, _ = run(case)
    r_out, _ = ref(case)
    assert_attention_close(out, r_out)
    case.indices = torch.from_numpy(idx[:, ::-1].copy()).to(DEV)
    out2, _ = run(case)
    assert_attention_close(out2, r_out)


def test_sparse_out_of_range_index_is_flagged_and_skipped():
    case = workloads.sparse_case(1, 16, 200, 40, device=DEV, seed=92)
    idx = npy(case.indices).copy()
    good = idx.copy()
    idx[0, 7] = 200
    idx[0, 30] = -5
    case.indices = torch.from_numpy(idx).to(DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _ = run(case, err_flag=flag)
    assert int(flag.item()) & dakv._lib.ERR_SPARSE_INDEX
    keep = [i for i in range(40) if i not in (7, 30)]
    r_out, _ = oracle.sparse_topk_decode(bits(case.q), bits(case.kv), good[:, keep],
                                         case.d_v, case.sm_scale)
    assert_attention_close(out, r_out)
    with pytest.raises(ValueError):
        dakv.validate_sparse(idx, 200)


def test_sparse_mla_full_size_every_sequence():
    """Batch 16, 128 heads, d_qk 576 / d_v 512, context 32768, top-2048: every output of
    every sequence against the oracle."""
    print("sparse full size", flush=True)
    case = workloads.sparse_mla(device=DEV, seed=5)
    out, lse = run(case)
    for b in range(16):
        r_out, r_lse = ref(case, rows=slice(b, b + 1))
        assert_attention_close(out[b:b + 1], r_out)
        assert_lse_close(lse[b:b + 1], r_lse)


# ------------------------------------------------------- several q-tokens per sequence


@pytest.mark.parametrize("B,s_q,Hq,s_kv,topk", [
    (2, 2, 16, 1000, 300),    # two tokens per sequence, two splits, ragged tile
    (1, 3, 32, 700, 65),      # three tokens, a ragged second tile
    (3, 2, 128, 4096, 2048),  # the config's heads and top-k, two tokens
    (2, 4, 16, 64, 1),        # a single index per token
])
def test_sparse_tokens_match_oracle(B, s_q, Hq, s_kv, topk):
    print(f"sparse tokens B={B} s_q={s_q} Hq={Hq} s_kv={s_kv} topk={topk}", flush=True)
    case = workloads.sparse_tokens_case(B, s_q, Hq, s_kv, topk, device=DEV, seed=60 + topk)
    out, lse = dakv.sparse_topk_attn(case.q, case.kv, case.indices, d_v=case.d_v,
                                     sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.sparse_topk_attn(bits(case.q), bits(case.kv), npy(case.indices),
                                           case.d_v, case.sm_scale)
    assert_attention_close(npy(out), r_out)
    assert_lse_close(npy(lse), r_lse)


def test_sparse_tokens_one_token_is_the_decode_call_and_bad_index_is_flagged():
    case = workloads.sparse_tokens_case(2, 1, 32, 500, 200, device=DEV, seed=67)
    o1, l1 = dakv.sparse_topk_attn(case.q, case.kv, case.indices, d_v=case.d_v,
                                   sm_scale=case.sm_scale)
    o2, l2 = dakv.sparse_topk_decode_attn(case.q[:, 0].contiguous(), case.kv,
                                          case.indices[:, 0].contiguous(), d_v=case.d_v,
                                          sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(l1[:, 0], l2)
    case = workloads.sparse_tokens_case(1, 2, 16, 200, 40, device=DEV, seed=68)
    idx = npy(case.indices).copy()
    good = idx.copy()
    idx[0, 1, 5] = 200                                 # token 1 only
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _ = dakv.sparse_topk_attn(case.q, case.kv, torch.from_numpy(idx).to(DEV),
                                   d_v=case.d_v, sm_scale=case.sm_scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_SPARSE_INDEX
    r0, _ = oracle.sparse_topk_attn(bits(case.q)[:, :1], bits(case.kv), good[:, :1],
                                    case.d_v, case.sm_scale)
    keep = [i for i in range(40) if i != 5]
    r1, _ = oracle.sparse_topk_attn(bits(case.q)[:, 1:], bits(case.kv), good[:, 1:, keep],
                                    case.d_v, case.sm_scale)
    assert_attention_close(npy(out)[:, :1], r0)
    assert_attention_close(npy(out)[:, 1:], r1)
