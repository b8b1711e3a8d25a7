"""Pins of the paged oracle (validation, gather_pa_kv_cache, paged GQA decode) -- CPU only."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import round_to_bf16_bits, widen
from oracle.paged import PagedIndexError
from conftest import bits

import workloads


def random_bits(rng, shape):
    return round_to_bf16_bits(rng.standard_normal(shape))


def any_bits(rng, shape):
    """Arbitrary 16-bit patterns (NaNs included): a copy must move any of them untouched.

    A multiplicative hash of the element index (random start) is used instead of a
    random draw so that the page's 5513-block pool fills quickly.
    """
    n = int(np.prod(shape))
    start = np.uint32(rng.integers(0, 1 << 31))
    x = np.arange(n, dtype=np.uint32)
    x += start
    x *= np.uint32(0x9E3779B1)
    x >>= np.uint32(16)
    return x.astype(np.uint16).reshape(shape)


# ---------------------------------------------------------------- hand-enumerated


def test_gather_hand_enumerated_two_sequences():
    """block_size 2, 5 physical blocks; every output row written out by hand.

    Sequence 0: 3 tokens, offset 2 (table column 1 onwards), table [9, 4, 1, 9].
      t=0 -> block 4 slot 0, t=1 -> block 4 slot 1, t=2 -> block 1 slot 0.
    Sequence 1: 2 tokens, no offset, table [3, 9, 9, 9].
      t=0 -> block 3 slot 0, t=1 -> block 3 slot 1.
    (9 marks entries that are never used; they are out of range on purpose.)
    """
    nb, bs = 5, 2
    kc = np.arange(nb * bs * 1 * 2, dtype=np.uint16).reshape(nb, bs, 1, 2)
    vc = (1000 + np.arange(nb * bs * 2 * 1, dtype=np.uint16)).reshape(nb, bs, 2, 1)
    tables = np.array([[9, 4, 1, 9], [3, 9, 9, 9]], dtype=np.int32)
    seq_lens = np.array([0, 3, 5], dtype=np.int32)
    offs = np.array([2, 0], dtype=np.int32)
    ko, vo = oracle.gather_pa_kv_cache(kc, vc, tables, seq_lens, offs)
    expect = [(4, 0), (4, 1), (1, 0), (3, 0), (3, 1)]
    assert ko.shape == (5, 1, 2) and vo.shape == (5, 2, 1)
    for row, (blk, slot) in enumerate(expect):
        assert np.array_equal(ko[row], kc[blk, slot])
        assert np.array_equal(vo[row], vc[blk, slot])


def test_gather_without_offset_equals_zero_offset():
    case = workloads.gather_case([5, 17, 0, 33], num_blocks=40, block_size=8, Hk=2, Dk=4,
                                 Hv=1, Dv=8, cols=6, seed=11, with_offset=False)
    kc, vc = bits(case.key_cache), bits(case.value_cache)
    a = oracle.gather_pa_kv_cache(kc, vc, case.index.block_tables, case.index.seq_lens, None)
    b = oracle.gather_pa_kv_cache(kc, vc, case.index.block_tables, case.index.seq_lens,
                                  np.zeros(4, dtype=np.int32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- inverse mapping


def test_scatter_then_gather_is_identity():
    """Write known contiguous rows into a pool through a table; the gather returns them."""
    rng = np.random.default_rng(12)
    lengths = [1, 7, 8, 9, 31, 0, 16]
    bs, Hk, Dk, Hv, Dv = 8, 3, 4, 2, 6
    index = workloads.gather_index(lengths, num_blocks=64, block_size=bs, cols=6, seed=13)
    T = sum(lengths)
    want_k = random_bits(rng, (T, Hk, Dk))
    want_v = random_bits(rng, (T, Hv, Dv))
    kc = random_bits(rng, (64, bs, Hk, Dk))
    vc = random_bits(rng, (64, bs, Hv, Dv))
    for q, L in enumerate(lengths):
        base = index.seq_lens[q]
        first = index.seq_offset[q] // bs
        for t in range(L):
            blk = index.block_tables[q, first + t // bs]
            kc[blk, t % bs] = want_k[base + t]
            vc[blk, t % bs] = want_v[base + t]
    ko, vo = oracle.gather_pa_kv_cache(kc, vc, index.block_tables, index.seq_lens,
                                       index.seq_offset)
    assert np.array_equal(ko, want_k) and np.array_equal(vo, want_v)


def test_block_relocation_leaves_gather_unchanged():
    case = workloads.gather_case([12, 40, 3], num_blocks=32, block_size=8, Hk=2, Dk=8,
                                 Hv=2, Dv=8, cols=8, seed=14)
    kc, vc = bits(case.key_cache), bits(case.value_cache)
    idx = case.index
    a = oracle.gather_pa_kv_cache(kc, vc, idx.block_tables, idx.seq_lens, idx.seq_offset)
    perm = np.random.default_rng(15).permutation(32)      # new home of block i is perm[i]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tables2 = perm[idx.block_tables].astype(np.int32)
    b = oracle.gather_pa_kv_cache(kc2, vc2, tables2, idx.seq_lens, idx.seq_offset)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------- printed shapes


def test_page_gather_shape_family(golden_dir):
    """The page's sweep (1 head, K dim 512 / V dim 64, block 128, 8 columns) and
    its two hand-picked shapes, rebuilt with our own seeded generator; checked
    against scatter-then-gather on shrunken pools (the printed pool of 5513 blocks
    is kept for one case)."""
    g = json.load(open(os.path.join(golden_dir, "gather_shapes.json")))
    sw = g["sweep"]
    nb_full, bs, Hk, Dk = sw["key_cache"]
    _, _, Hv, Dv = sw["value_cache"]
    for i, c in enumerate(sw["cases"]):
        Q, T = c["Q"], c["T"]
        rng = np.random.default_rng(100 + i)
        cut = np.sort(rng.choice(np.arange(1, T), Q - 1, replace=False))
        lengths = np.diff(np.concatenate([[0], cut, [T]])).tolist()
        nb = nb_full if i == 0 else 64
        index = workloads.gather_index(lengths, num_blocks=nb, block_size=bs,
                                       cols=sw["block_table_cols"], seed=200 + i)
        kc = any_bits(rng, (nb, bs, Hk, Dk))
        vc = any_bits(rng, (nb, bs, Hv, Dv))
        ko, vo = oracle.gather_pa_kv_cache(kc, vc, index.block_tables, index.seq_lens,
                                           index.seq_offset)
        assert ko.shape == (T, Hk, Dk) and vo.shape == (T, Hv, Dv)
        for q, L in enumerate(lengths):
            base, first = index.seq_lens[q], index.seq_offset[q] // bs
            for t in range(L):
                blk = index.block_tables[q, first + t // bs]
                assert np.array_equal(ko[base + t], kc[blk, t % bs])
                assert np.array_equal(vo[base + t], vc[blk, t % bs])
    for m in g["manual"]:
        nb, bs, Hk, Dk = m["key_cache"]
        _, _, Hv, Dv = m["value_cache"]
        T = m["key_out"][0]
        rng = np.random.default_rng(16)
        index = workloads.gather_index([2, 4], num_blocks=nb, block_size=bs, cols=4, seed=16)
        kc, vc = any_bits(rng, (nb, bs, Hk, Dk)), any_bits(rng, (nb, bs, Hv, Dv))
        ko, vo = oracle.gather_pa_kv_cache(kc, vc, index.block_tables, index.seq_lens,
                                           index.seq_offset)
        assert list(ko.shape) == m["key_out"] and list(vo.shape) == m["value_out"]
        assert T == 6
        for q, L in enumerate([2, 4]):
            for t in range(L):
                blk = index.block_tables[q, index.seq_offset[q] // bs + t // bs]
                assert np.array_equal(ko[index.seq_lens[q] + t], kc[blk, t % bs])


# ------------------------------------------------------------------ validation


def _ok_index():
    tables = np.array([[0, 1, 2], [3, 4, 5]], dtype=np.int32)
    return tables, np.array([0, 5, 9], dtype=np.int32), np.array([0, 2], dtype=np.int32)


def test_validation_accepts_a_good_index():
    t, s, o = _ok_index()
    oracle.validate_paged(t, s, o, num_blocks=6, block_size=2)


@pytest.mark.parametrize("bad", [
    "not_cumsum_length", "nonzero_start", "decreasing", "negative_offset",
    "unaligned_offset", "block_id_high", "block_id_negative", "beyond_table",
])
def test_validation_rejects(bad):
    t, s, o = _ok_index()
    if bad == "not_cumsum_length":
        s = np.array([5, 4], dtype=np.int32)          # per-sequence lengths, not cumulative
    elif bad == "nonzero_start":
        s = np.array([1, 5, 9], dtype=np.int32)
    elif bad == "decreasing":
        s = np.array([0, 5, 4], dtype=np.int32)
    elif bad == "negative_offset":
        o = np.array([-2, 0], dtype=np.int32)
    elif bad == "unaligned_offset":
        o = np.array([1, 0], dtype=np.int32)
    elif bad == "block_id_high":
        t = t.copy(); t[0, 1] = 6
    elif bad == "block_id_negative":
        t = t.copy(); t[1, 2] = -1
    elif bad == "beyond_table":
        o = np.array([0, 4], dtype=np.int32)          # columns 2..3 of a 3-column table
    with pytest.raises(PagedIndexError):
        oracle.validate_paged(t, s, o, num_blocks=6, block_size=2)


def test_unused_table_entries_are_not_validated():
    t, s, o = _ok_index()
    t = t.copy()
    t[0, 2] = -7          # sequence 0 (5 tokens, bs 2, offset 0) uses columns 0..2 -> bad
    with pytest.raises(PagedIndexError):
        oracle.validate_paged(t, s, o, num_blocks=6, block_size=2)
    s2 = np.array([0, 4, 8], dtype=np.int32)          # now only columns 0..1 are used
    oracle.validate_paged(t, s2, o, num_blocks=6, block_size=2)


# ------------------------------------------------------------ paged attention


def test_paged_equals_static_layout_on_the_same_rows():
    """The same K/V, once in the static layout and once paged, give equal results."""
    lengths = [1, 17, 48, 5]
    Hq, Hkv, D, bs = 4, 2, 8, 16
    case = workloads.paged_case(lengths, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, seed=17)
    kc, vc, qb = bits(case.key_cache), bits(case.value_cache), bits(case.q)
    out_p, lse_p = oracle.decode_paged(qb, kc, vc, case.index.block_tables,
                                       case.index.seq_lens, None)
    cap = max(lengths)
    group = Hq // Hkv
    Ks = np.zeros((len(lengths), Hq, cap, D), dtype=np.uint16)
    Vs = np.zeros_like(Ks)
    for b, L in enumerate(lengths):
        for t in range(L):
            blk = case.index.block_tables[b, t // bs]
            for h in range(Hq):
                Ks[b, h, t] = kc[blk, t % bs, h // group]
                Vs[b, h, t] = vc[blk, t % bs, h // group]
    out_s, lse_s = oracle.decode_static(widen(qb), Ks, Vs, valid_len=lengths)
    assert np.allclose(out_p, out_s, rtol=0, atol=1e-14)
    assert np.allclose(lse_p, lse_s, rtol=0, atol=1e-13)


def test_table_walk_equals_gather_then_dense():
    lengths = [33, 2, 64, 19]
    case = workloads.paged_case(lengths, Hq=8, Hkv=2, D=16, block_size=16, seed=18)
    args = (bits(case.q), bits(case.key_cache), bits(case.value_cache),
            case.index.block_tables, case.index.seq_lens, None)
    a = oracle.decode_paged(*args)
    b = oracle.decode_paged_via_gather(*args)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-14)
    assert np.allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_gqa_group_mapping_uses_contiguous_query_heads():
    """Give KV head 1 a distinctive constant V; query heads 2, 3 (of 4, 2 KV heads)
    must return it, heads 0, 1 must not."""
    lengths = [9]
    case = workloads.paged_case(lengths, Hq=4, Hkv=2, D=4, block_size=4, seed=19)
    vc = bits(case.value_cache).copy()
    vc[:, :, 1, :] = round_to_bf16_bits(np.full(4, 3.0))
    out, _ = oracle.decode_paged(bits(case.q), bits(case.key_cache), vc,
                                 case.index.block_tables, case.index.seq_lens, None)
    assert np.allclose(out[0, 2:], 3.0, atol=1e-14)
    assert not np.allclose(out[0, :2], 3.0, atol=1e-3)


def test_paged_single_token_and_empty_sequence():
    lengths = [1, 0]
    case = workloads.paged_case(lengths, Hq=2, Hkv=1, D=8, block_size=16, seed=20)
    kc, vc = bits(case.key_cache), bits(case.value_cache)
    out, lse = oracle.decode_paged(bits(case.q), kc, vc, case.index.block_tables,
                                   case.index.seq_lens, None)
    blk = case.index.block_tables[0, 0]
    assert np.array_equal(out[0, 0], widen(vc[blk, 0, 0]))
    assert np.all(out[1] == 0) and np.all(lse[1] == -math.inf)
