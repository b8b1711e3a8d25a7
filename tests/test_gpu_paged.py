"""GPU parity: gather_pa_kv_cache (bit-exact) and decode_attn_paged vs the fp64 oracle."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(index):
    t = torch.from_numpy(index.block_tables).to(DEV)
    s = torch.from_numpy(index.seq_lens).to(DEV)
    o = None if index.seq_offset is None else torch.from_numpy(index.seq_offset).to(DEV)
    return t, s, o


def gather_and_check(case):
    t, s, o = to_dev(case.index)
    ko, vo = dakv.gather_pa_kv_cache(case.key_cache, case.value_cache, t, s, o)
    torch.cuda.synchronize()
    ek, ev = oracle.gather_pa_kv_cache(bits(case.key_cache), bits(case.value_cache),
                                       case.index.block_tables, case.index.seq_lens,
                                       case.index.seq_offset)
    assert np.array_equal(bits(ko), ek)
    assert np.array_equal(bits(vo), ev)


@pytest.mark.parametrize("bs", [16, 128])
def test_gather_ragged_bit_exact(bs):
    lengths = [1, bs - 1, bs, bs + 1, 0, 3 * bs + 7]
    case = workloads.gather_case(lengths, num_blocks=64, block_size=bs, Hk=8, Dk=128, Hv=8,
                                 Dv=128, cols=8, device=DEV, seed=40)
    gather_and_check(case)


def test_gather_page_shape_family(golden_dir):
    """Shapes printed on the PyPTO page: 1 head with K dim 512 / V dim 64, block 128,
    8 table columns, T up to 55; and the 64-head x 128 case."""
    g = json.load(open(os.path.join(golden_dir, "gather_shapes.json")))
    nb, bs, Hk, Dk = g["sweep"]["key_cache"]
    _, _, Hv, Dv = g["sweep"]["value_cache"]
    for i, c in enumerate(g["sweep"]["cases"]):
        rng = np.random.default_rng(41 + i)
        cut = np.sort(rng.choice(np.arange(1, c["T"]), c["Q"] - 1, replace=False))
        lengths = np.diff(np.concatenate([[0], cut, [c["T"]]])).tolist()
        case = workloads.gather_case(lengths, num_blocks=nb if i == 0 else 128, block_size=bs,
                                     Hk=Hk, Dk=Dk, Hv=Hv, Dv=Dv,
                                     cols=g["sweep"]["block_table_cols"], device=DEV,
                                     seed=41 + i)
        gather_and_check(case)
    for m in g["manual"]:
        nb, bs, Hk, Dk = m["key_cache"]
        _, _, Hv, Dv = m["value_cache"]
        case = workloads.gather_case([2, 4], num_blocks=nb, block_size=bs, Hk=Hk, Dk=Dk, Hv=Hv,
                                     Dv=Dv, cols=4, device=DEV, seed=60)
        gather_and_check(case)


def test_gather_full_size_bit_exact():
    """key/value cache [8192, 128, 8, 128], 32 sequences of 1..4096 tokens."""
    print("gather full size", flush=True)
    case = workloads.gather_nd(device=DEV, seed=3)
    gather_and_check(case)


def test_gather_bad_block_id_is_flagged_and_zeroed():
    case = workloads.gather_case([5, 9], num_blocks=16, block_size=4, Hk=1, Dk=64, Hv=1, Dv=64,
                                 cols=4, device=DEV, seed=43, with_offset=False)
    tables = case.index.block_tables.copy()
    tables[1, 1] = 99                      # tokens 4..7 of sequence 1
    t = torch.from_numpy(tables).to(DEV)
    s = torch.from_numpy(case.index.seq_lens).to(DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ko, vo = dakv.gather_pa_kv_cache(case.key_cache, case.value_cache, t, s, None,
                                     err_flag=flag, validate=False)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_BLOCK_ID
    kb = bits(ko)
    assert np.all(kb[5 + 4:5 + 8] == 0)
    good = list(range(0, 9)) + [13]
    tables[1, 1] = case.index.block_tables[1, 1]
    ek, _ = oracle.gather_pa_kv_cache(bits(case.key_cache), bits(case.value_cache), tables,
                                      case.index.seq_lens, None)
    assert np.array_equal(kb[good], ek[good])


def test_gather_block_relocation_invariance():
    case = workloads.gather_case([40, 3, 77], num_blocks=48, block_size=16, Hk=2, Dk=64, Hv=4,
                                 Dv=32, cols=8, device=DEV, seed=44)
    t, s, o = to_dev(case.index)
    k1, v1 = dakv.gather_pa_kv_cache(case.key_cache, case.value_cache, t, s, o)
    perm = torch.from_numpy(np.random.default_rng(45).permutation(48)).to(DEV)
    kc2 = torch.empty_like(case.key_cache)
    vc2 = torch.empty_like(case.value_cache)
    kc2[perm] = case.key_cache
    vc2[perm] = case.value_cache
    t2 = perm[t.long()].to(torch.int32)
    k2, v2 = dakv.gather_pa_kv_cache(kc2, vc2, t2, s, o)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))


# ---------------------------------------------------------------- paged decode


def run_paged(case, **kw):
    t, s, o = to_dev(case.index)
    out, lse = dakv.decode_attn_paged(case.q, case.key_cache, case.value_cache, t, s, o,
                                      scale=case.scale, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


def oracle_paged(case):
    return oracle.decode_paged(bits(case.q), bits(case.key_cache), bits(case.value_cache),
                               case.index.block_tables, case.index.seq_lens,
                               case.index.seq_offset, case.scale)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_paged_gqa_groups_match_oracle(G):
    lengths = [1, 15, 16, 17, 100, 513, 0, 1000]
    case = workloads.paged_case(lengths, Hq=2 * G, Hkv=2, D=128, block_size=16, device=DEV,
                                seed=50 + G)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (64, 8), (16, 16), (32, 16), (16, 4),
                                     (6, 3), (24, 3), (32, 32)])
def test_paged_head_layouts_match_oracle(Hq, Hkv):
    """KV head counts that divide 16 (one workgroup reads whole token rows of all
    heads) and ones that do not (one workgroup per KV head)."""
    lengths = [1, 15, 16, 17, 100, 513, 0, 700]
    case = workloads.paged_case(lengths, Hq=Hq, Hkv=Hkv, D=128, block_size=16, device=DEV,
                                seed=80 + Hq + Hkv)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_paged_block_sizes_with_offsets(bs):
    lengths = [3 * bs + 5, bs, 1, 700]
    case = workloads.paged_case(lengths, Hq=8, Hkv=2, D=128, block_size=bs, device=DEV,
                                seed=60 + bs)
    # shift every sequence's table by one column via seq_offset
    idx = case.index
    cols = idx.block_tables.shape[1]
    shifted = np.full((len(lengths), cols + 1), -1, dtype=np.int32)
    shifted[:, 1:] = idx.block_tables
    idx.block_tables = shifted
    idx.seq_offset = np.full(len(lengths), bs, dtype=np.int32)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_paged_single_token_bit_exact_and_empty_sequence():
    case = workloads.paged_case([1, 0, 1], Hq=4, Hkv=1, D=128, block_size=16, device=DEV,
                                seed=70)
    out, lse = run_paged(case)
    vc = bits(case.value_cache)
    for b in (0, 2):
        blk = case.index.block_tables[b, 0]
        expect = (vc[blk, 0, 0].astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(out[b], np.broadcast_to(expect, out[b].shape))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_paged_block_relocation_bit_identical():
    case = workloads.paged_case([200, 31, 64], Hq=8, Hkv=2, D=128, block_size=16, device=DEV,
                                seed=71)
    out1, lse1 = run_paged(case)
    nb = case.index.num_blocks
    perm = np.random.default_rng(72).permutation(nb)
    pt = torch.from_numpy(perm).to(DEV)
    kc2 = torch.empty_like(case.key_cache)
    vc2 = torch.empty_like(case.value_cache)
    kc2[pt] = case.key_cache
    vc2[pt] = case.value_cache
    tables = case.index.block_tables
    case.index.block_tables = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    case.key_cache, case.value_cache = kc2, vc2
    out2, lse2 = run_paged(case)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_paged_split_counts_agree():
    case = workloads.paged_case([3000, 1200], Hq=8, Hkv=2, D=128, block_size=16, device=DEV,
                                seed=73)
    out_a, _ = run_paged(case)
    out_1, _ = run_paged(case, num_splits=1)
    out_9, _ = run_paged(case, num_splits=9)
    assert np.max(np.abs(out_a - out_1)) <= 1e-5 * np.max(np.abs(out_1))
    assert np.max(np.abs(out_9 - out_1)) <= 1e-5 * np.max(np.abs(out_1))


def test_paged_bad_block_id_is_flagged():
    case = workloads.paged_case([40, 40], Hq=4, Hkv=1, D=128, block_size=16, device=DEV,
                                seed=74)
    case.index.block_tables[1, 1] = 10 ** 6
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _ = run_paged(case, err_flag=flag)
    assert int(flag.item()) & dakv._lib.ERR_BLOCK_ID
    # sequence 0 is unaffected
    case.index.block_tables[1, 1] = case.index.block_tables[1, 0]
    ref, _ = oracle_paged(case)
    assert_attention_close(out[0], ref[0])


def test_paged_gqa_full_size_every_sequence():
    """Batch 64, 32/8 heads, block 16, contexts log-uniform on [512, 16384]; every
    output of every sequence against the oracle."""
    print("paged full size", flush=True)
    case = workloads.paged_gqa(device=DEV, seed=4)
    out, lse = run_paged(case)
    kc, vc, qb = bits(case.key_cache), bits(case.value_cache), bits(case.q)
    idx = case.index
    for b in range(64):
        L = idx.lengths[b]
        ref_out, ref_lse = oracle.decode_paged(qb[b:b + 1], kc, vc, idx.block_tables[b:b + 1],
                                               np.array([0, L], dtype=np.int32), None,
                                               case.scale)
        assert_attention_close(out[b:b + 1], ref_out)
        assert_lse_close(lse[b:b + 1], ref_lse)


def test_paged_longest_supported_sequence():
    """Block 16: 256 splits of 1024 tokens = 262144 tokens is the longest sequence the
    paged kernel takes; one token more is refused on the host."""
    print("paged 262144 tokens", flush=True)
    case = workloads.paged_case([262144, 3], Hq=4, Hkv=1, D=128, block_size=16, device=DEV,
                                seed=77)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
    t, s, o = to_dev(case.index)
    with pytest.raises(ValueError):
        dakv.decode_attn_paged(case.q, case.key_cache, case.value_cache, t, s, o,
                               max_seq_len=262145)


# ---------------------------------------------- the matrix-core kernel's own edges
# (Hkv in {2, 4, 8k} with D = 128 and at most 512 sequences take paged_mfma_kernel;
# the tests above with one or three KV heads reach the other kernels)

def test_paged_mfma_ranges_cut_groups_and_workspace_reuse():
    """The matrix-core kernel gives every workgroup an equal range of 16-token tiles, so
    ranges cut through (sequence, head group) pairs: mixed lengths (empty and one-token
    sequences among them) with many pieces per group; then the same workspace for a call
    with other piece counts, and for one whose sequences all fit a single split (no
    merge, the recorded piece counts of the earlier calls left in the workspace)."""
    calls = ([5000, 0, 1, 3000, 17, 12000, 640], [40000, 33, 2048], [300, 0, 511])
    need = max(dakv.decode_attn_paged_workspace_size(len(c), 32, 128, max(c), 16) for c in calls)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for i, lengths in enumerate(calls):
        print(f"paged ranges call {i}: {lengths}", flush=True)
        case = workloads.paged_case(lengths, Hq=32, Hkv=8, D=128, block_size=16, device=DEV,
                                    seed=180 + i)
        out, lse = run_paged(case, workspace=ws)
        ref_out, ref_lse = oracle_paged(case)
        assert_attention_close(out, ref_out)
        assert_lse_close(lse, ref_lse)


def test_paged_mfma_single_token_bit_exact_and_empty_sequence():
    case = workloads.paged_case([1, 0, 1], Hq=8, Hkv=2, D=128, block_size=16, device=DEV,
                                seed=170)
    out, lse = run_paged(case)
    vc = bits(case.value_cache)
    for b in (0, 2):
        blk = case.index.block_tables[b, 0]
        for h in range(8):
            expect = (vc[blk, 0, h // 4].astype(np.uint32) << 16).view(np.float32)
            assert np.array_equal(out[b, h], expect), (b, h)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_paged_mfma_bad_block_id_is_flagged_and_others_unaffected():
    case = workloads.paged_case([40, 40, 300], Hq=32, Hkv=8, D=128, block_size=16, device=DEV,
                                seed=174)
    good = case.index.block_tables.copy()
    case.index.block_tables[1, 1] = 10 ** 6
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _ = run_paged(case, err_flag=flag)
    assert int(flag.item()) & dakv._lib.ERR_BLOCK_ID
    case.index.block_tables = good
    ref, _ = oracle_paged(case)
    assert_attention_close(out[0], ref[0])
    assert_attention_close(out[2], ref[2])


@pytest.mark.parametrize("B", [512, 513])
def test_paged_sequence_count_at_the_split_map_limit(B):
    """512 sequences are the most the matrix-core kernel's split map holds (one more
    takes the all-heads kernel); both against the oracle."""
    print(f"paged B={B}", flush=True)
    rng = np.random.default_rng(180 + B)
    lengths = rng.integers(0, 40, size=B).tolist()
    case = workloads.paged_case(lengths, Hq=32, Hkv=8, D=128, block_size=16, device=DEV,
                                seed=181 + B)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_paged_mfma_longest_supported_sequence():
    """Block 16, 2 KV heads: 262144 tokens (256 splits of 1024) through the matrix-core
    kernel, with a 3-token sequence beside it."""
    print("paged mfma 262144 tokens", flush=True)
    case = workloads.paged_case([262144, 3], Hq=2, Hkv=2, D=128, block_size=16, device=DEV,
                                seed=177)
    out, lse = run_paged(case)
    ref_out, ref_lse = oracle_paged(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
