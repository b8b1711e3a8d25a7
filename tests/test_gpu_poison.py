"""GPU: garbage in cache slots outside the attended set never reaches the output.

The NPU article's static-buffer design ("Solution: preallocation + attention mask")
turns every masked slot into -inf before the softmax, so the slot is ignored
completely, and its section on padding side effects warns that those slots hold
garbage.  Here every slot that no attended row names -- masked rows and rows past the
valid length of the static caches; unused pool blocks (block 0 among them), the tail
slots of each sequence's last block and the block a bad table entry points away from
in the paged pools -- is filled with NaN, +-Inf or N(0, 100^2) values (NaN codes and
infinite or NaN row scales in the FP8 and FP4 caches), and every output bit must stay
as it was.  The clean run is also checked against the oracle.
"""

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
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(
        torch.bfloat16)


# ------------------------------------------------------------------------ paged pools


def block0_unused(index):
    """The same index with pool block 0 moved to an id no sequence uses (the unused
    row loads of a kernel that re-read a fixed pool location would land there)."""
    t = index.block_tables.copy()
    used = set(int(x) for x in t[t >= 0])
    if 0 in used:
        free = next(i for i in range(index.num_blocks) if i not in used)
        t[t == 0] = free
    return workloads.PagedIndex(t, index.seq_lens, index.seq_offset, index.lengths,
                                index.num_blocks, index.block_size)


def named_slots(index):
    """bool [num_blocks, block_size]: True where token t < len_b of some sequence b
    lives (table entries outside the pool name nothing)."""
    nb, bs = index.num_blocks, index.block_size
    named = np.zeros((nb, bs), dtype=bool)
    offs = index.seq_offset if index.seq_offset is not None else np.zeros(len(index.lengths),
                                                                          np.int64)
    for b, L in enumerate(index.lengths):
        for t in range(L):
            phys = int(index.block_tables[b, offs[b] // bs + t // bs])
            if 0 <= phys < nb:
                named[phys, t % bs] = True
    return named


def poison_bf16(shape, kind, rng):
    if kind == "nan":
        x = np.full(shape, np.nan)
    elif kind == "inf":
        x = np.full(shape, np.inf)
        x.reshape(-1)[::2] = -np.inf
    else:
        x = rng.standard_normal(shape) * 100.0
    return round_to_bf16_bits(x)


def lowbit_poison(fmt, kind):
    """(code byte, scale) written into every unnamed slot of an FP8 / FP4 pool."""
    code = {"fp8": 0x7F if kind == "nan" else 0xFF,   # the two E4M3 NaN codes
            "fp4": 0x77 if kind == "nan" else 0xFF}[fmt]  # +-6 in both nibbles
    return code, (np.nan if kind == "nan" else np.inf)


def paged_tensors(index, **arrays):
    t = torch.from_numpy(index.block_tables).to(DEV)
    s = torch.from_numpy(index.seq_lens).to(DEV)
    o = None if index.seq_offset is None else torch.from_numpy(index.seq_offset).to(DEV)
    return t, s, o


PAGED_SHAPES = [
    # lengths, Hq, Hkv, bs
    ([1, 100, 700, 33], 8, 8, 16),     # G = 1
    ([1, 100, 700, 33], 8, 2, 16),     # G = 4
    ([129, 17, 250], 32, 8, 16),       # the paged config's heads
    ([300, 64, 5], 16, 4, 128),        # G = 4, block 128
]


@pytest.mark.parametrize("kind", ["nan", "inf", "sigma100"])
@pytest.mark.parametrize("lengths,Hq,Hkv,bs", PAGED_SHAPES + [([90, 400], 12, 3, 16)])
def test_paged_bf16_unnamed_slots_are_bit_invisible(lengths, Hq, Hkv, bs, kind):
    """bf16 pool (the last shape, 3 KV heads, runs the one-head-per-workgroup kernel)."""
    print(f"poison paged bf16 {lengths} Hq={Hq} Hkv={Hkv} bs={bs} {kind}", flush=True)
    rng = np.random.default_rng(600 + Hq + bs)
    D = 128
    index = block0_unused(workloads.pool_index(lengths, block_size=bs, slack=0.3, seed=601))
    shape = (index.num_blocks, bs, Hkv, D)
    kc = round_to_bf16_bits(rng.standard_normal(shape))
    vc = round_to_bf16_bits(rng.standard_normal(shape))
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    t, s, o = paged_tensors(index)

    def run(k, v, **kw):
        out, lse = dakv.decode_attn_paged(bf16_dev(q), bf16_dev(k), bf16_dev(v), t, s, o, **kw)
        torch.cuda.synchronize()
        return npy(out), npy(lse)

    clean = [run(kc, vc), run(kc, vc, num_splits=5)]
    ref_out, ref_lse = oracle.decode_paged(q, kc, vc, index.block_tables, index.seq_lens,
                                           None, 1.0 / np.sqrt(D))
    assert_attention_close(clean[0][0], ref_out)
    assert_lse_close(clean[0][1], ref_lse)
    dead = ~named_slots(index)
    assert dead[0].all()
    kp, vp = kc.copy(), vc.copy()
    kp[dead] = poison_bf16(kp[dead].shape, kind, rng)
    vp[dead] = poison_bf16(vp[dead].shape, kind, rng)
    for (o0, l0), kw in zip(clean, [{}, {"num_splits": 5}]):
        o1, l1 = run(kp, vp, **kw)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), kw


@pytest.mark.parametrize("kind", ["nan", "inf"])
def test_paged_bf16_bad_block_id_is_skipped_and_garbage_stays_invisible(kind):
    """A table entry outside the pool: its rows are skipped (error bit), the block the
    entry used to name is unnamed and poisoned, and nothing else changes."""
    rng = np.random.default_rng(610)
    lengths, Hq, Hkv, bs, D = [1, 100, 700, 33], 8, 2, 16, 128
    index = block0_unused(workloads.pool_index(lengths, block_size=bs, slack=0.3, seed=611))
    index.block_tables[2, 3] = index.num_blocks + 7
    shape = (index.num_blocks, bs, Hkv, D)
    kc = round_to_bf16_bits(rng.standard_normal(shape))
    vc = round_to_bf16_bits(rng.standard_normal(shape))
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    t, s, o = paged_tensors(index)

    def run(k, v):
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        out, lse = dakv.decode_attn_paged(bf16_dev(q), bf16_dev(k), bf16_dev(v), t, s, o,
                                          err_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) & dakv._lib.ERR_BLOCK_ID
        return npy(out), npy(lse)

    o0, l0 = run(kc, vc)
    dead = ~named_slots(index)
    kp, vp = kc.copy(), vc.copy()
    kp[dead] = poison_bf16(kp[dead].shape, kind, rng)
    vp[dead] = poison_bf16(vp[dead].shape, kind, rng)
    o1, l1 = run(kp, vp)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # the other sequences are the oracle's
    keep = [0, 1, 3]
    sub = workloads.pool_index([lengths[i] for i in keep], block_size=bs, slack=0.0, seed=0)
    sub.block_tables[:] = index.block_tables[keep][:, :sub.block_tables.shape[1]]
    ref, _ = oracle.decode_paged(q[keep], kc, vc, sub.block_tables, sub.seq_lens, None,
                                 1.0 / np.sqrt(D))
    assert_attention_close(o0[keep], ref)


def lowbit_pool(fmt, rng, nb, bs, Hkv, D):
    per = 2 if fmt == "fp4" else 1
    shape = (nb, bs, Hkv, D // per)
    codes = []
    for _ in range(2):
        c = rng.integers(0, 256, size=shape).astype(np.uint8)
        if fmt == "fp8":
            c[(c & 0x7F) == 0x7F] = 0x7E
        codes.append(c)
    lo, hi = (-12, -5) if fmt == "fp8" else (-3, 1)
    scales = [np.exp2(rng.integers(lo, hi, size=shape[:3])).astype(np.float32) for _ in range(2)]
    return [codes[0], codes[1], scales[0], scales[1]]


@pytest.mark.parametrize("kind", ["nan", "inf"])
@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("lengths,Hq,Hkv,bs", PAGED_SHAPES)
def test_paged_lowbit_unnamed_slots_are_bit_invisible(fmt, lengths, Hq, Hkv, bs, kind):
    print(f"poison paged {fmt} {lengths} Hq={Hq} Hkv={Hkv} bs={bs} {kind}", flush=True)
    rng = np.random.default_rng(620 + Hq + bs)
    D = 128
    index = block0_unused(workloads.pool_index(lengths, block_size=bs, slack=0.3, seed=621))
    pool = lowbit_pool(fmt, rng, index.num_blocks, bs, Hkv, D)
    q = round_to_bf16_bits(rng.standard_normal((len(lengths), Hq, D)))
    t, s, o = paged_tensors(index)
    fn = dakv.decode_attn_paged_fp8 if fmt == "fp8" else dakv.decode_attn_paged_fp4

    def run(arrays, **kw):
        dev = [torch.from_numpy(a).to(DEV) for a in arrays]
        out, lse = fn(bf16_dev(q), *dev, t, s, o, **kw)
        torch.cuda.synchronize()
        return npy(out), npy(lse)

    clean = [run(pool), run(pool, num_splits=5)]
    ref_fn = oracle.decode_paged_fp8 if fmt == "fp8" else oracle.decode_paged_fp4
    ref_out, ref_lse = ref_fn(q, *pool, index.block_tables, index.seq_lens)
    assert_attention_close(clean[0][0], ref_out)
    assert_lse_close(clean[0][1], ref_lse)
    dead = ~named_slots(index)
    assert dead[0].all()
    code, sc = lowbit_poison(fmt, kind)
    bad = [a.copy() for a in pool]
    for a in bad[:2]:
        a[dead] = code
    for a in bad[2:]:
        a[dead] = sc
    for (o0, l0), kw in zip(clean, [{}, {"num_splits": 5}]):
        o1, l1 = run(bad, **kw)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), kw


# ----------------------------------------------------------------------- static caches


def static_dead_rows(mask, lengths, cap):
    """bool [B, cap]: masked rows below the valid length and every row at or past it."""
    dead = np.ones((len(lengths), cap), dtype=bool)
    for b, L in enumerate(lengths):
        dead[b, :L] = mask[b, :L] == 0
    return dead


STATIC_SHAPES = [
    # B, H, D, cap, lengths
    (3, 4, 128, 700, [700, 450, 37]),
    (2, 3, 64, 1152, [103, 1100]),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kind", ["nan", "inf"])
@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("B,H,D,cap,lengths", STATIC_SHAPES)
def test_static_lowbit_unattended_rows_are_bit_invisible(B, H, D, cap, lengths, fmt, kind,
                                                         fused):
    """FP8 / FP4 static caches: NaN codes and infinite or NaN K and V row scales in
    masked rows and rows at or past the valid length; with the fused step the new row
    L - 1 (mask entry 0 before the step) is poisoned too and overwritten by the
    append."""
    print(f"poison static {fmt} B={B} D={D} cap={cap} {kind} fused={fused}", flush=True)
    rng = np.random.default_rng(640 + D + cap)
    per = 2 if fmt == "fp4" else 1
    shape = (B, H, cap, D // per)
    codes = [rng.integers(0, 256, size=shape).astype(np.uint8) for _ in range(2)]
    if fmt == "fp8":
        for c in codes:
            c[(c & 0x7F) == 0x7F] = 0x7E
    lo, hi = (-12, -5) if fmt == "fp8" else (-3, 1)
    scales = [np.exp2(rng.integers(lo, hi, size=(B, H, cap))).astype(np.float32)
              for _ in range(2)]
    mask = np.zeros((B, cap), np.int32)
    for b, L in enumerate(lengths):
        mask[b, :L] = rng.uniform(size=L) < 0.8
    pos = np.array([L - 1 for L in lengths], np.int32)
    if fused:
        mask[np.arange(B), pos] = 0
    q = (rng.standard_normal((B, H, D)) * (0.05 if fmt == "fp8" else 0.3)).astype(np.float32)
    kn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    vn = round_to_bf16_bits(rng.standard_normal((B, H, D)))
    vl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    if fmt == "fp8":
        attn, step, app = (dakv.decode_attn_static_fp8, dakv.decode_step_static_fp8,
                           dakv.kv_append_fp8)
    else:
        attn, step, app = (dakv.decode_attn_static_fp4, dakv.decode_step_static_fp4,
                           dakv.kv_append_fp4)

    def run(arrays, two_calls=False):
        kc, vc, ks, vs = [torch.from_numpy(a.copy()).to(DEV) for a in arrays]
        m = torch.from_numpy(mask.copy()).to(DEV)
        qd = torch.from_numpy(q).to(DEV)
        p = torch.from_numpy(pos).to(DEV)
        if not fused:
            out, lse = attn(qd, kc, vc, ks, vs, mask=m, valid_len=vl)
        elif two_calls:
            app(kc, vc, ks, vs, bf16_dev(kn), bf16_dev(vn), p, mask=m)
            out, lse = attn(qd, kc, vc, ks, vs, mask=m, valid_len=vl)
        else:
            out, lse = step(qd, kc, vc, ks, vs, bf16_dev(kn), bf16_dev(vn), p, mask=m,
                            valid_len=vl)
        torch.cuda.synchronize()
        return npy(out), npy(lse)

    clean = codes + scales
    o0, l0 = run(clean)
    dead = static_dead_rows(mask, lengths, cap)
    code, sc = lowbit_poison(fmt, kind)
    bad = [a.copy() for a in clean]
    for a in bad[:2]:
        a.transpose(0, 2, 1, 3)[dead] = code
    for a in bad[2:]:
        a.transpose(0, 2, 1)[dead] = sc
    o1, l1 = run(bad)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    if fused:
        o2, l2 = run(bad, two_calls=True)
        assert np.array_equal(o0, o2) and np.array_equal(l0, l2)
        if fmt == "fp8":
            ref_c = oracle.kv_append_fp8(*[a.copy() for a in clean], kn, vn, pos, mask.copy())
            ref_out, ref_lse = oracle.decode_static_fp8(q, *ref_c[:4], ref_c[4], lengths)
        else:
            ref_c = oracle.kv_append_fp4(*[a.copy() for a in clean], kn, vn, pos, mask.copy())
            ref_out, ref_lse = oracle.decode_static_fp4(q, *ref_c[:4], ref_c[4], lengths)
    else:
        ref_fn = oracle.decode_static_fp8 if fmt == "fp8" else oracle.decode_static_fp4
        ref_out, ref_lse = ref_fn(q, *clean, mask, lengths)
    assert_attention_close(o0, ref_out)
    assert_lse_close(l0, ref_lse)


@pytest.mark.parametrize("kind", ["nan", "inf", "sigma100"])
def test_static_bf16_fused_step_unattended_rows_are_bit_invisible(kind):
    """decode_step_static: garbage in masked rows and rows past the valid length (the
    new row's slot included, which the append overwrites) changes no output bit."""
    rng = np.random.default_rng(660)
    B, H, D, cap, lengths = 3, 4, 128, 700, [700, 450, 37]
    case = workloads.static_case(B, H, D, cap, lengths, device=DEV, seed=661,
                                 mask_density=0.8)
    pos = torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device=DEV)
    case.mask[torch.arange(B), pos.long()] = 0
    g = torch.Generator(device=DEV).manual_seed(662)
    kn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)

    def run(k, v):
        k, v, m = k.clone(), v.clone(), case.mask.clone()
        out, lse = dakv.decode_step_static(case.q, k, v, kn, vn, pos, mask=m,
                                           valid_len=case.valid_len, scale=case.scale)
        torch.cuda.synchronize()
        return npy(out), npy(lse)

    o0, l0 = run(case.k_cache, case.v_cache)
    dead = torch.from_numpy(static_dead_rows(npy(case.mask), lengths, cap)).to(DEV)
    sel = dead[:, None, :, None].expand_as(case.k_cache)
    junk = bf16_dev(poison_bf16(tuple(case.k_cache.shape), kind, rng))
    kp, vp = case.k_cache.clone(), case.v_cache.clone()
    kp[sel] = junk[sel]
    vp[sel] = junk[sel]
    o1, l1 = run(kp, vp)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    ek, ev, em = oracle.kv_append(bits(case.k_cache), bits(case.v_cache), bits(kn), bits(vn),
                                  npy(pos), npy(case.mask))
    ref_out, ref_lse = oracle.decode_static(npy(case.q), ek, ev, em, lengths, case.scale)
    assert_attention_close(o0, ref_out)
    assert_lse_close(l0, ref_lse)
