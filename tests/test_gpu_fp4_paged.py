"""GPU parity: the FP4 paged pool (E2M1 codes two per byte) -- quantising append of each
sequence's new last token (codes and scales bit-exact) and paged GQA decode over the codes
(within the attention tolerance) vs the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, npy
from oracle import round_to_bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_dev(bits_u16):
    return torch.from_numpy(bits_u16.view(np.int16)).to(DEV).view(torch.bfloat16)


def fp4_pool(rng, nb, bs, Hkv, D):
    """Random bytes (two finite E2M1 codes each) [nb, bs, Hkv, D / 2]; row scales
    2^-3 .. 2^0 (those of O(1) rows)."""
    shape = (nb, bs, Hkv, D // 2)
    codes = [rng.integers(0, 256, size=shape).astype(np.uint8) for _ in range(2)]
    scales = [np.exp2(rng.integers(-3, 1, size=shape[:3])).astype(np.float32) for _ in range(2)]
    return codes[0], codes[1], scales[0], scales[1]


def run_decode(q_bits, pool, index, **kw):
    t = torch.from_numpy(index.block_tables).to(DEV)
    s = torch.from_numpy(index.seq_lens).to(DEV)
    o = None if index.seq_offset is None else torch.from_numpy(index.seq_offset).to(DEV)
    dev = [torch.from_numpy(a).to(DEV) for a in pool]
    out, lse = dakv.decode_attn_paged_fp4(bf16_dev(q_bits), *dev, t, s, o, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


@pytest.mark.parametrize("lengths,Hq,Hkv,bs", [
    ([1, 100, 700], 8, 2, 16),            # G = 4, ragged blocks and splits
    ([513, 2000], 32, 8, 16),             # the config's heads
    ([5, 64, 65, 1000], 4, 4, 32),        # G = 1
    ([300, 1], 16, 2, 64),                # G = 8
    ([129, 0, 77], 8, 4, 128),            # an empty sequence, block 128
    ([700, 33], 32, 16, 16),              # 16 KV heads: several head groups
    ([40, 300], 4, 1, 16),                # one KV head: the VALU kernel
])
def test_paged_fp4_decode_matches_oracle(lengths, Hq, Hkv, bs):
    print(f"paged fp4 lengths={lengths} Hq={Hq} Hkv={Hkv} bs={bs}", flush=True)
    rng = np.random.default_rng(300 + bs + Hq)
    D = 128
    index = workloads.pool_index(lengths, block_size=bs, slack=0.1, seed=201 + bs)
    pool = fp4_pool(rng, index.num_blocks, bs, Hkv, D)
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    out, lse = run_decode(q, pool, index)
    ref_out, ref_lse = oracle.decode_paged_fp4(q, *pool, index.block_tables, index.seq_lens)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
    many, _ = run_decode(q, pool, index, num_splits=37)
    assert_attention_close(many, ref_out)


def test_paged_fp4_decode_with_table_offsets():
    rng = np.random.default_rng(310)
    lengths, bs, Hkv, Hq, D = [1, 300, 127, 128], 16, 2, 8, 128
    index = workloads.gather_index(lengths, num_blocks=160, block_size=bs, cols=40, seed=211)
    pool = fp4_pool(rng, index.num_blocks, bs, Hkv, D)
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    out, lse = run_decode(q, pool, index)
    ref_out, ref_lse = oracle.decode_paged_fp4(q, *pool, index.block_tables, index.seq_lens,
                                               index.seq_offset)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


def test_paged_append_fp4_bit_exact_then_attended():
    rng = np.random.default_rng(320)
    lengths, bs, Hkv, Hq, D = [1, 16, 17, 500], 16, 4, 16, 128
    index = workloads.pool_index(lengths, block_size=bs, slack=0.1, seed=221)
    pool = fp4_pool(rng, index.num_blocks, bs, Hkv, D)
    kn = round_to_bf16_bits(rng.standard_normal((len(lengths), Hkv, D)) * 4)
    vn = round_to_bf16_bits(rng.standard_normal((len(lengths), Hkv, D)) * 0.02)
    want = oracle.paged_append_fp4(*pool, kn, vn, index.block_tables, index.seq_lens)
    dev = [torch.from_numpy(a).to(DEV) for a in pool]
    t = torch.from_numpy(index.block_tables).to(DEV)
    s = torch.from_numpy(index.seq_lens).to(DEV)
    dakv.paged_append_fp4(*dev, bf16_dev(kn), bf16_dev(vn), t, s)
    torch.cuda.synchronize()
    got = [npy(x) for x in dev]
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert np.array_equal(got[2].astype(np.float64), want[2])
    assert np.array_equal(got[3].astype(np.float64), want[3])
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    out, _ = dakv.decode_attn_paged_fp4(bf16_dev(q), *dev, t, s)
    torch.cuda.synchronize()
    ref_out, _ = oracle.decode_paged_fp4(q, *want, index.block_tables, index.seq_lens)
    assert_attention_close(npy(out), ref_out)


def test_paged_append_fp4_flags_empty_sequence_and_bad_block():
    rng = np.random.default_rng(330)
    bs, Hkv, D = 16, 2, 128
    index = workloads.pool_index([5, 20], block_size=bs, slack=0.1, seed=231)
    pool = fp4_pool(rng, index.num_blocks, bs, Hkv, D)
    kn = round_to_bf16_bits(rng.standard_normal((3, Hkv, D)))
    tables = np.concatenate([index.block_tables, np.full((1, index.block_tables.shape[1]), -1,
                                                         np.int32)])
    tables[0, 0] = index.num_blocks + 5                       # bad id for sequence 0
    seq_lens = np.array([0, 5, 25, 25], np.int32)             # sequence 2 is empty
    dev = [torch.from_numpy(a).to(DEV) for a in pool]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.paged_append_fp4(*dev, bf16_dev(kn), bf16_dev(kn), torch.from_numpy(tables).to(DEV),
                          torch.from_numpy(seq_lens).to(DEV), err_flag=flag)
    torch.cuda.synchronize()
    f = int(flag.item())
    assert f & dakv._lib.ERR_BLOCK_ID and f & dakv._lib.ERR_SEQ_LENS
    # only sequence 1's last token (position 19) changed
    p, sl = index.block_tables[1, 19 // bs], 19 % bs
    got = npy(dev[0])
    mask = np.ones(got.shape[:2], bool)
    mask[p, sl] = False
    assert np.array_equal(got[mask], pool[0][mask])
    qk, _ = oracle.fp4.quantize_rows(kn[1])
    assert np.array_equal(got[p, sl], qk)


def test_paged_fp4_full_size_every_sequence():
    """Batch 64, 32 query / 8 KV heads, block 16, contexts log-uniform [512, 16384], FP4
    pool: every sequence against the oracle."""
    print("paged fp4 full size", flush=True)
    rng = np.random.default_rng(340)
    lengths = workloads.log_uniform_lengths(64, 512, 16384, 4)
    index = workloads.pool_index(lengths, block_size=16, slack=0.1, seed=4)
    pool = fp4_pool(rng, index.num_blocks, 16, 8, 128)
    q = round_to_bf16_bits(rng.standard_normal((64, 32, 128)))
    out, lse = run_decode(q, pool, index)
    for b in range(64):
        sub = workloads.PagedIndex(index.block_tables[b:b + 1],
                                   np.array([0, lengths[b]], np.int32), None, [lengths[b]],
                                   index.num_blocks, 16)
        r_out, r_lse = oracle.decode_paged_fp4(q[b:b + 1], *pool, sub.block_tables, sub.seq_lens)
        assert_attention_close(out[b:b + 1], r_out)
        assert_lse_close(lse[b:b + 1], r_lse)
