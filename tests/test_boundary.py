"""The C-ABI boundary on the CPU: the library loads, exports every declared entry
point, and its host-side checks and validators reject what the contract rejects.
No call here reaches the GPU: every one returns from a host check first."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oracle.paged import PagedIndexError

import decode_attention_kv_amd as dakv
from decode_attention_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dakv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dakv_\w+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = declared_functions()
    assert len(names) >= 12
    lib = dakv.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_texts():
    for code in (0, -1, -2, -3, -4):
        assert dakv.strerror(code)
    assert dakv.strerror(0) == "ok"


# ------------------------------------------------------------- host validators


def _paged_cases(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        Q = int(rng.integers(1, 6))
        bs = int(rng.choice([1, 2, 4, 16]))
        cols = int(rng.integers(1, 6))
        nb = int(rng.integers(1, 40))
        lens = rng.integers(0, bs * cols + 1, size=Q)
        seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        tables = rng.integers(-2, nb + 2, size=(Q, cols)).astype(np.int32)
        offs = (bs * rng.integers(0, cols, size=Q)).astype(np.int32)
        kind = rng.integers(0, 6)
        if kind == 1:
            offs[0] += 1                       # unaligned
        elif kind == 2:
            seq[1:] = seq[1:][::-1].copy()     # may decrease
        elif kind == 3:
            seq[0] = 1
        elif kind == 4:
            offs[-1] = -bs
        yield tables, seq, (None if kind == 5 else offs), nb, bs


def test_validate_paged_agrees_with_the_oracle():
    n_ok = n_bad = 0
    for tables, seq, offs, nb, bs in _paged_cases(40):
        try:
            oracle.validate_paged(tables, seq, offs, nb, bs)
            expect_ok = True
        except PagedIndexError:
            expect_ok = False
        if expect_ok:
            dakv.validate_paged(tables, seq, offs, nb, bs)
            n_ok += 1
        else:
            with pytest.raises(ValueError):
                dakv.validate_paged(tables, seq, offs, nb, bs)
            n_bad += 1
    assert n_ok > 5 and n_bad > 5


def test_validate_paged_rejects_non_cumulative_seq_lens():
    with pytest.raises(ValueError, match="cumulative"):
        dakv.validate_paged(np.zeros((2, 3), np.int32), np.array([3, 4], np.int32), None, 4, 2)


def test_validate_sparse_and_range():
    dakv.validate_sparse(np.array([[0, 5, 9]], np.int32), 10)
    for bad in (-1, 10):
        with pytest.raises(ValueError):
            dakv.validate_sparse(np.array([[0, bad]], np.int32), 10)
    dakv.validate_range(np.array([0, 3, 7], np.int32), 0, 7)
    with pytest.raises(ValueError):
        dakv.validate_range(np.array([0, 8], np.int32), 0, 7)


# ------------------------------------------------------- argument checks (no GPU)

NULL = None


def test_entry_points_reject_bad_arguments_before_any_launch():
    L = dakv.lib()
    fake = ctypes.c_void_p(4096)       # aligned, never dereferenced: the checks fail first
    odd = ctypes.c_void_p(4096 + 8)    # misaligned
    # kv_append: null cache, negative sizes, D*2 not a multiple of 16
    assert L.dakv_kv_append(NULL, fake, fake, fake, fake, NULL, 1, 1, 4, 8, NULL, NULL) == _lib.EINVAL
    assert L.dakv_kv_append(fake, fake, fake, fake, fake, NULL, -1, 1, 4, 8, NULL, NULL) == _lib.EINVAL
    assert L.dakv_kv_append(fake, fake, fake, fake, fake, NULL, 1, 1, 4, 4, NULL, NULL) == _lib.ENOTSUP
    assert L.dakv_kv_append(odd, fake, fake, fake, fake, NULL, 1, 1, 4, 8, NULL, NULL) == _lib.EINVAL
    # empty batch is a no-op success
    assert L.dakv_kv_append(NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 4, 8, NULL, NULL) == _lib.OK
    # decode_attn_static: unsupported D, neither mask nor valid_len, short workspace
    ws = L.dakv_decode_attn_static_workspace_size(1, 4, 1152, 64)
    assert ws > 0
    args = lambda D, mask, vl, wsb: (fake, fake, fake, mask, vl, 1, 4, 1152, D, 0.125, fake,
                                     NULL, fake, wsb, 0, NULL, NULL)
    assert L.dakv_decode_attn_static(*args(96, fake, NULL, ws)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_static(*args(64, NULL, NULL, ws)) == _lib.EINVAL
    assert L.dakv_decode_attn_static(*args(64, fake, NULL, ws - 4)) == _lib.EINVAL
    # gather: odd row bytes, zero tables
    assert L.dakv_gather_pa_kv_cache(fake, fake, 8, 4, 1, 3, 1, 8, fake, 1, 2, fake, NULL, 4,
                                     fake, fake, NULL, NULL) == _lib.ENOTSUP
    assert L.dakv_gather_pa_kv_cache(fake, fake, 8, 4, 1, 8, 1, 8, fake, 0, 2, fake, NULL, 4,
                                     fake, fake, NULL, NULL) == _lib.EINVAL
    assert L.dakv_gather_pa_kv_cache(fake, fake, 8, 4, 1, 8, 1, 8, fake, 1, 2, fake, NULL, 0,
                                     fake, fake, NULL, NULL) == _lib.OK
    # paged: heads not divisible, unsupported block size / head dim
    wsp = L.dakv_decode_attn_paged_workspace_size(2, 8, 128, 100, 16)
    pargs = lambda Hq, Hkv, D, bs: (fake, fake, fake, fake, 4, fake, NULL, 2, Hq, Hkv, D, 10, bs,
                                    100, 0.1, fake, NULL, fake, wsp, 0, NULL, NULL)
    assert L.dakv_decode_attn_paged(*pargs(8, 3, 128, 16)) == _lib.EINVAL
    assert L.dakv_decode_attn_paged(*pargs(8, 2, 128, 12)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_paged(*pargs(8, 2, 64, 16)) == _lib.ENOTSUP
    # copy_kvcache: no tensors, too many, a null or misaligned tensor pointer, odd rows
    ptrs = lambda *p: ctypes.cast((ctypes.c_void_p * len(p))(*p), ctypes.c_void_p)
    two = ptrs(4096, 8192)
    cargs = lambda src, dst, n, D: (src, dst, n, 1, 2, 16, 20, D, fake, NULL, NULL, NULL)
    assert L.dakv_copy_kvcache(*cargs(two, two, 0, 8)) == _lib.EINVAL
    assert L.dakv_copy_kvcache(*cargs(two, two, _lib.COPY_MAX_TENSORS + 1, 8)) == _lib.EINVAL
    assert L.dakv_copy_kvcache(*cargs(ptrs(4096, 0), two, 2, 8)) == _lib.EINVAL
    assert L.dakv_copy_kvcache(*cargs(two, ptrs(4096, 8200), 2, 8)) == _lib.EINVAL
    assert L.dakv_copy_kvcache(*cargs(two, two, 2, 4)) == _lib.ENOTSUP
    assert L.dakv_copy_kvcache(NULL, NULL, 1, 0, 2, 16, 20, 8, NULL, NULL, NULL, NULL) == _lib.OK
    # fp8: unsupported head dims, missing scales
    assert L.dakv_kv_append_fp8(fake, fake, fake, fake, fake, fake, fake, NULL, 1, 1, 4, 24,
                                NULL, NULL) == _lib.ENOTSUP
    assert L.dakv_kv_append_fp8(fake, fake, NULL, fake, fake, fake, fake, NULL, 1, 1, 4, 64,
                                NULL, NULL) == _lib.EINVAL
    wsf = L.dakv_decode_attn_static_fp8_workspace_size(1, 4, 1152, 64)
    assert wsf == L.dakv_decode_attn_static_workspace_size(1, 4, 1152, 64)
    fargs = lambda D, ksc: (fake, fake, fake, ksc, fake, fake, NULL, 1, 4, 1152, D, 0.125, fake,
                            NULL, fake, wsf, 0, NULL, NULL)
    assert L.dakv_decode_attn_static_fp8(*fargs(96, fake)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_static_fp8(*fargs(64, NULL)) == _lib.EINVAL
    # trim_kvcache: null mask, bad capacity
    assert L.dakv_trim_kvcache(NULL, fake, 1, 8, NULL, NULL) == _lib.EINVAL
    assert L.dakv_trim_kvcache(fake, fake, 1, 0, NULL, NULL) == _lib.EINVAL
    # sparse: unsupported dims
    assert L.dakv_sparse_topk_decode_attn(fake, fake, fake, 1, 128, 100, 256, 128, 8, 0.1, fake,
                                          NULL, fake, 1 << 20, NULL, NULL) == _lib.ENOTSUP


def test_low_bit_fused_and_sparse_entry_points_reject_bad_arguments():
    """Host checks of the FP8/FP4, fused-step, latent-append and sparse entry points:
    each bad argument returns its status before anything is launched."""
    L = dakv.lib()
    fake = ctypes.c_void_p(4096)
    ws = L.dakv_decode_attn_static_workspace_size(1, 4, 1152, 64)
    # kv_append_fp4: D not a multiple of 16, missing write position
    assert L.dakv_kv_append_fp4(*([fake] * 7), NULL, 1, 1, 4, 24, NULL, NULL) == _lib.ENOTSUP
    assert L.dakv_kv_append_fp4(*([fake] * 6), NULL, NULL, 1, 1, 4, 64, NULL, NULL) == _lib.EINVAL
    # decode_attn_static_fp4: head dim, missing scales, short workspace
    f4 = lambda D, ksc, wsb: (fake, fake, fake, ksc, fake, fake, NULL, 1, 4, 1152, D, 0.125,
                              fake, NULL, fake, wsb, 0, NULL, NULL)
    assert L.dakv_decode_attn_static_fp4(*f4(96, fake, ws)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_static_fp4(*f4(64, NULL, ws)) == _lib.EINVAL
    assert L.dakv_decode_attn_static_fp4(*f4(64, fake, ws - 4)) == _lib.EINVAL
    # fused steps (bf16, FP8, FP4): head dim, missing write position, neither mask nor
    # valid length, short workspace, capacity past the largest split plan
    low = lambda D, wp, m, vl, wsb, cap=1152: (fake, fake, fake, fake, fake, fake, fake, wp, m,
                                               vl, 1, 4, cap, D, 0.125, fake, NULL, fake, wsb, 0,
                                               NULL, NULL)
    bf = lambda D, wp, m, vl, wsb, cap=1152: (fake, fake, fake, fake, fake, wp, m, vl, 1, 4, cap,
                                              D, 0.125, fake, NULL, fake, wsb, 0, NULL, NULL)
    for fn, args in ((L.dakv_decode_step_static_fp8, low), (L.dakv_decode_step_static_fp4, low),
                     (L.dakv_decode_step_static, bf)):
        assert fn(*args(96, fake, fake, NULL, ws)) == _lib.ENOTSUP
        assert fn(*args(64, NULL, fake, NULL, ws)) == _lib.EINVAL
        assert fn(*args(64, fake, NULL, NULL, ws)) == _lib.EINVAL
        assert fn(*args(64, fake, fake, NULL, ws - 4)) == _lib.EINVAL
        assert fn(*args(64, fake, fake, NULL, ws, 1 << 20)) == _lib.ENOTSUP
    # paged FP4 append: head dim, no table columns, missing table
    pa = lambda tab, cols, D: (fake, fake, fake, fake, fake, fake, tab, cols, fake, NULL, 2, 2, D,
                               10, 16, NULL, NULL)
    assert L.dakv_paged_append_fp4(*pa(fake, 4, 24)) == _lib.ENOTSUP
    assert L.dakv_paged_append_fp4(*pa(fake, 0, 128)) == _lib.EINVAL
    assert L.dakv_paged_append_fp4(*pa(NULL, 4, 128)) == _lib.EINVAL
    # paged FP4 decode: heads not divisible, head dim, group of 16, block size
    wsp = L.dakv_decode_attn_paged_workspace_size(2, 64, 128, 100, 16)
    pd = lambda Hq, Hkv, D, bs: (fake, fake, fake, fake, fake, fake, 4, fake, NULL, 2, Hq, Hkv, D,
                                 10, bs, 100, 0.1, fake, NULL, fake, wsp, 0, NULL, NULL)
    assert L.dakv_decode_attn_paged_fp4(*pd(8, 3, 128, 16)) == _lib.EINVAL
    assert L.dakv_decode_attn_paged_fp4(*pd(8, 2, 64, 16)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_paged_fp4(*pd(64, 4, 128, 16)) == _lib.ENOTSUP
    assert L.dakv_decode_attn_paged_fp4(*pd(8, 2, 128, 12)) == _lib.ENOTSUP
    # latent appends: rows longer than 576, odd FP4 rows, missing scales, empty batch
    la = lambda sc, d: (fake, sc, fake, fake, 2, 64, d, NULL, NULL)
    assert L.dakv_latent_append_fp8(*la(fake, 600)) == _lib.ENOTSUP
    assert L.dakv_latent_append_fp4(*la(fake, 577)) == _lib.ENOTSUP
    assert L.dakv_latent_append_fp4(*la(NULL, 576)) == _lib.EINVAL
    assert L.dakv_latent_append_fp8(NULL, NULL, NULL, NULL, 0, 64, 576, NULL, NULL) == _lib.OK
    # sparse over codes: missing scales, head count, latent width, a cache too long for
    # 32-bit row offsets, too many (sequence, token) pairs; empty batch is a no-op
    sp = lambda sc, B, s_q, Hq, s_kv, d_qk: (fake, fake, sc, fake, B, s_q, Hq, s_kv, d_qk, 512,
                                             64, 0.04, fake, NULL, fake, 1 << 30, NULL, NULL)
    for fn in (L.dakv_sparse_topk_attn_fp8, L.dakv_sparse_topk_attn_fp4):
        assert fn(*sp(NULL, 1, 1, 128, 4096, 576)) == _lib.EINVAL
        assert fn(*sp(fake, 1, 1, 24, 4096, 576)) == _lib.ENOTSUP
        assert fn(*sp(fake, 1, 1, 128, 4096, 512)) == _lib.ENOTSUP
        assert fn(*sp(fake, 1, 1, 128, 2_000_000, 576)) == _lib.ENOTSUP
        assert fn(*sp(fake, 1 << 13, 1 << 12, 128, 4096, 576)) == _lib.EINVAL
        assert fn(*sp(NULL, 0, 1, 128, 4096, 576)) == _lib.OK
    # several q-tokens (bf16): no tokens is a no-op, a missing index table is an error
    st = lambda s_q, idx: (fake, fake, idx, 1, s_q, 128, 4096, 576, 512, 64, 0.04, fake, NULL,
                           fake, 1 << 30, NULL, NULL)
    assert L.dakv_sparse_topk_attn(*st(0, NULL)) == _lib.OK
    assert L.dakv_sparse_topk_attn(*st(2, NULL)) == _lib.EINVAL


def test_python_binding_rejects_cpu_tensors():
    import torch
    k = torch.zeros((1, 1, 4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        dakv.decode_attn_static(torch.zeros((1, 1, 8)), k, k, valid_len=torch.ones(1, dtype=torch.int32))


def test_static_split_rows_query_names_the_instantiation():
    """Host planning of the static split pass (rows per split) as the kernels use it:
    a call of the LLaMA-7B-shaped layer at batch 8 takes 128-row splits, at batch 1
    64-row ones; forced split counts and large capacities take up to 256 rows."""
    rows = dakv.decode_attn_static_split_rows
    assert rows(8, 32, 4096, 128) == 128
    assert rows(1, 32, 4096, 128) == 64
    assert rows(4, 4, 4096, 128) == 64
    assert rows(8, 32, 4096, 128, num_splits=32) == 128
    assert rows(1, 4, 4096, 128, num_splits=1) == 256
    assert rows(2, 2, 65536, 64) == 256
    assert rows(1, 1, 65537, 64) == 0
    assert rows(1, 1, 4096, 96) == 0


def test_noalloc_entry_checks_its_scratch_limit_on_the_host():
    """The allocation-free decode_attn_static form reports the partial bytes a call
    needs and refuses, before any device work, calls beyond its fixed scratch."""
    L = dakv.lib()
    need = L.dakv_decode_attn_static_noalloc_scratch_bytes
    assert need(8, 32, 4096, 128, 0) == 8 * 32 * 32 * 129 * 4   # 128-row splits
    assert need(1, 4, 256, 128, 1) == 0                          # one split: no partials
    assert need(1, 1, 4096, 96, 0) == 0                          # unsupported head_dim
    fake = ctypes.c_void_p(4096)
    args = lambda B, H, cap: (fake, fake, fake, NULL, fake, B, H, cap, 128, 0.1, fake, NULL, 0,
                              NULL, NULL)
    assert need(64, 32, 4096, 128, 0) > _lib.NOALLOC_SCRATCH_BYTES
    assert L.dakv_decode_attn_static_noalloc(*args(64, 32, 4096)) == _lib.ESCRATCH
    assert L.dakv_decode_attn_static_noalloc(*args(0, 32, 4096)) == _lib.OK
    assert L.dakv_decode_attn_static_noalloc(NULL, fake, fake, NULL, fake, 1, 1, 64, 128, 0.1,
                                             fake, NULL, 0, NULL, NULL) == _lib.EINVAL
    assert "scratch" in dakv.strerror(_lib.ESCRATCH)
