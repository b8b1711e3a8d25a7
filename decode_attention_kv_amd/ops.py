"""Thin torch-facing binding of the C-ABI (argument marshalling only).

Every function here has the name of its C entry point without the ``dakv_`` prefix.
torch is used for device memory (outputs and workspace are allocated with it when
the caller does not pass them) and for the current stream; all computation
happens in the HIP kernels of libdakv.so.  Shape/dtype/device mistakes raise
``ValueError`` before any call; a nonzero C status raises ``DakvError`` (a
``ValueError``).
"""

import ctypes
import math

import numpy as np
import torch

from . import _lib
from ._lib import COPY_MAX_TENSORS, check, lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _opt(t, name, dtype, shape=None):
    return None if t is None else _need(t, name, dtype, shape)


def _host_i32(x):
    """A host int32 numpy copy of an index tensor (a device copy synchronises)."""
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu")
        return np.ascontiguousarray(x.numpy().astype(np.int32, copy=False))
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _hp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ validators


def validate_paged(block_tables, seq_lens, seq_offset, num_blocks, block_size):
    """Host check of paged index content (cumulative seq_lens, offsets, block ids)."""
    t = _host_i32(block_tables)
    if t.ndim != 2:
        raise ValueError("block_tables must be [Q, cols]")
    s = _host_i32(seq_lens).reshape(-1)
    Q, cols = t.shape
    if s.shape != (Q + 1,):
        raise ValueError("only cumulative seq_lens of length Q + 1 is supported")
    o = None if seq_offset is None else _host_i32(seq_offset).reshape(-1)
    if o is not None and o.shape != (Q,):
        raise ValueError("seq_offset must be [Q]")
    check("validate_paged", lib().dakv_validate_paged(_hp(t), Q, cols, _hp(s), _hp(o),
                                                      int(num_blocks), int(block_size)))


def validate_sparse(indices, s_kv):
    a = _host_i32(indices)
    B, topk = a.shape if a.ndim == 2 else (1, a.size)
    check("validate_sparse", lib().dakv_validate_sparse(_hp(a), B, topk, int(s_kv)))


def validate_range(values, lo, hi):
    a = _host_i32(values).reshape(-1)
    check("validate_range", lib().dakv_validate_range(_hp(a), a.size, int(lo), int(hi)))


# ------------------------------------------------------------------- kv_append


def kv_append(k_cache, v_cache, k_new, v_new, write_pos, mask=None, err_flag=None):
    """Write k_new/v_new [B, H, D] into row write_pos[b] of k_cache/v_cache [B, H, cap, D]."""
    _need(k_cache, "k_cache", torch.bfloat16)
    B, H, cap, D = k_cache.shape
    _need(v_cache, "v_cache", torch.bfloat16, (B, H, cap, D))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("kv_append", lib().dakv_kv_append(_p(k_cache), _p(v_cache), _p(k_new), _p(v_new),
                                            _p(write_pos), _p(mask), B, H, cap, D,
                                            _p(err_flag), _stream()))


# ------------------------------------------------------------- fp8 KV cache


def kv_append_fp8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos, mask=None,
                  err_flag=None):
    """Quantise k_new/v_new bf16 [B, H, D] to E4M3 codes with a power-of-two scale per
    row and store them at row write_pos[b] of k_codes/v_codes uint8 [B, H, cap, D]
    and k_scale/v_scale fp32 [B, H, cap]."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, D = k_codes.shape
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, D))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("kv_append_fp8", lib().dakv_kv_append_fp8(
        _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(k_new), _p(v_new),
        _p(write_pos), _p(mask), B, H, cap, D, _p(err_flag), _stream()))


def decode_attn_static_fp8(q, k_codes, v_codes, k_scale, v_scale, mask=None, valid_len=None,
                           scale=None, out=None, lse=None, workspace=None, num_splits=0,
                           err_flag=None, want_lse=True):
    """decode_attn_static over an FP8 cache (uint8 E4M3 codes [B, H, cap, D] and fp32
    row scales [B, H, cap] for K and V).  Returns ``(out, lse)``."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, D = k_codes.shape
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, D))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(q, "q", torch.float32, (B, H, D))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = int(lib().dakv_decode_attn_static_fp8_workspace_size(B, H, cap, D))
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_attn_static_fp8", lib().dakv_decode_attn_static_fp8(
        _p(q), _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(mask), _p(valid_len),
        B, H, cap, D, float(scale), _p(out), _p(lse), _p(ws), ws.numel(), int(num_splits),
        _p(err_flag), _stream()))
    return out, lse


def kv_append_fp4(k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos, mask=None,
                  err_flag=None):
    """Quantise k_new/v_new bf16 [B, H, D] to E2M1 codes (two per byte) with a
    power-of-two scale per row and store them at row write_pos[b] of k_codes/v_codes
    uint8 [B, H, cap, D/2] and k_scale/v_scale fp32 [B, H, cap]."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, half = k_codes.shape
    D = 2 * half
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, half))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("kv_append_fp4", lib().dakv_kv_append_fp4(
        _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(k_new), _p(v_new),
        _p(write_pos), _p(mask), B, H, cap, D, _p(err_flag), _stream()))


def decode_attn_static_fp4(q, k_codes, v_codes, k_scale, v_scale, mask=None, valid_len=None,
                           scale=None, out=None, lse=None, workspace=None, num_splits=0,
                           err_flag=None, want_lse=True):
    """decode_attn_static over an FP4 cache (uint8 [B, H, cap, D/2], two E2M1 codes per
    byte, element 2i in the low four bits; fp32 row scales [B, H, cap]).  Returns
    ``(out, lse)``."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, half = k_codes.shape
    D = 2 * half
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, half))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(q, "q", torch.float32, (B, H, D))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = decode_attn_static_workspace_size(B, H, cap, D)
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_attn_static_fp4", lib().dakv_decode_attn_static_fp4(
        _p(q), _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(mask), _p(valid_len),
        B, H, cap, D, float(scale), _p(out), _p(lse), _p(ws), ws.numel(), int(num_splits),
        _p(err_flag), _stream()))
    return out, lse


def decode_step_static_fp8(q, k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos,
                           mask=None, valid_len=None, scale=None, out=None, lse=None,
                           workspace=None, num_splits=0, err_flag=None, want_lse=True):
    """kv_append_fp8 followed by decode_attn_static_fp8, in one pass.  Returns
    ``(out, lse)``."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, D = k_codes.shape
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, D))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(q, "q", torch.float32, (B, H, D))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = int(lib().dakv_decode_attn_static_fp8_workspace_size(B, H, cap, D))
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_step_static_fp8", lib().dakv_decode_step_static_fp8(
        _p(q), _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(k_new), _p(v_new),
        _p(write_pos), _p(mask), _p(valid_len), B, H, cap, D, float(scale), _p(out), _p(lse),
        _p(ws), ws.numel(), int(num_splits), _p(err_flag), _stream()))
    return out, lse


def decode_step_static_fp4(q, k_codes, v_codes, k_scale, v_scale, k_new, v_new, write_pos,
                           mask=None, valid_len=None, scale=None, out=None, lse=None,
                           workspace=None, num_splits=0, err_flag=None, want_lse=True):
    """kv_append_fp4 followed by decode_attn_static_fp4, in one pass (codes uint8
    [B, H, cap, D / 2]).  Returns ``(out, lse)``."""
    _need(k_codes, "k_codes", torch.uint8)
    B, H, cap, half = k_codes.shape
    D = 2 * half
    _need(v_codes, "v_codes", torch.uint8, (B, H, cap, half))
    _need(k_scale, "k_scale", torch.float32, (B, H, cap))
    _need(v_scale, "v_scale", torch.float32, (B, H, cap))
    _need(q, "q", torch.float32, (B, H, D))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = int(lib().dakv_decode_attn_static_fp8_workspace_size(B, H, cap, D))
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_step_static_fp4", lib().dakv_decode_step_static_fp4(
        _p(q), _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(k_new), _p(v_new),
        _p(write_pos), _p(mask), _p(valid_len), B, H, cap, D, float(scale), _p(out), _p(lse),
        _p(ws), ws.numel(), int(num_splits), _p(err_flag), _stream()))
    return out, lse


# ------------------------------------------------------ copy_kvcache / trim


def copy_kvcache(src, dst, lengths, mask=None, err_flag=None):
    """Copy rows [0, lengths[b]) of every src[i] [B, H, S_src, D] into dst[i]
    [B, H, S_dst, D] (the prefill -> generate hand-over); other dst rows are kept.
    When ``mask`` [B, S_dst] is given it becomes 1 for the copied rows, 0 after."""
    src, dst = list(src), list(dst)
    if not src or len(src) != len(dst):
        raise ValueError("src and dst must be equally long, non-empty lists")
    if len(src) > COPY_MAX_TENSORS:
        raise ValueError(f"at most {COPY_MAX_TENSORS} tensor pairs per call")
    if src[0].dim() != 4:
        raise ValueError("tensors must be [B, H, S, D]")
    B, H, S_src, D = src[0].shape
    S_dst = dst[0].shape[2] if dst[0].dim() == 4 else -1
    dtype = src[0].dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("tensors must be bf16 or fp16")
    for i, (s_t, d_t) in enumerate(zip(src, dst)):
        _need(s_t, f"src[{i}]", dtype, (B, H, S_src, D))
        _need(d_t, f"dst[{i}]", dtype, (B, H, S_dst, D))
    _need(lengths, "lengths", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, S_dst))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    n = len(src)
    src_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src])
    dst_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst])
    check("copy_kvcache", lib().dakv_copy_kvcache(
        ctypes.cast(src_arr, ctypes.c_void_p), ctypes.cast(dst_arr, ctypes.c_void_p), n, B, H,
        S_src, S_dst, D, _p(lengths), _p(mask), _p(err_flag), _stream()))


def trim_kvcache(mask, new_len, err_flag=None):
    """Rows at and after new_len[b] of mask [B, cap] stop counting (set to 0)."""
    _need(mask, "mask", torch.int32)
    if mask.dim() != 2:
        raise ValueError("mask must be [B, cap]")
    B, cap = mask.shape
    _need(new_len, "new_len", torch.int32, (B,))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("trim_kvcache", lib().dakv_trim_kvcache(_p(mask), _p(new_len), B, cap, _p(err_flag),
                                                  _stream()))


# ---------------------------------------------------------- decode_attn_static


def decode_attn_static_workspace_size(B, H, cap, D):
    return int(lib().dakv_decode_attn_static_workspace_size(B, H, cap, D))


def decode_attn_static_split_rows(B, H, cap, D, num_splits=0):
    """Rows per split of a static-layout decode call of these sizes (0: unsupported)."""
    return int(lib().dakv_decode_attn_static_split_rows(B, H, cap, D, num_splits))


def _workspace(nbytes, device, workspace):
    """The caller's workspace, or a new one."""
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def decode_attn_static(q, k_cache, v_cache, mask=None, valid_len=None, scale=None, out=None,
                       lse=None, workspace=None, num_splits=0, err_flag=None, want_lse=True):
    """Decode attention over the static buffer.  Returns ``(out, lse)``.

    q fp32 [B, H, D]; k_cache/v_cache bf16 [B, H, cap, D]; mask int32 [B, cap] and/or
    valid_len int32 [B].  ``lse`` is None when ``want_lse`` is false and no lse
    tensor is given.
    """
    _need(k_cache, "k_cache", torch.bfloat16)
    B, H, cap, D = k_cache.shape
    _need(v_cache, "v_cache", torch.bfloat16, (B, H, cap, D))
    _need(q, "q", torch.float32, (B, H, D))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = decode_attn_static_workspace_size(B, H, cap, D)
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_attn_static", lib().dakv_decode_attn_static(
        _p(q), _p(k_cache), _p(v_cache), _p(mask), _p(valid_len), B, H, cap, D, float(scale),
        _p(out), _p(lse), _p(ws), ws.numel(), int(num_splits), _p(err_flag), _stream()))
    return out, lse


def decode_attn_static_noalloc(q, k_cache, v_cache, mask=None, valid_len=None, scale=None,
                               out=None, lse=None, num_splits=0, err_flag=None, want_lse=True):
    """decode_attn_static with its split partials in the library's fixed device scratch
    (no workspace argument; the C call allocates nothing).  Returns ``(out, lse)``.
    Calls that overlap on one GPU share that scratch and must not run concurrently."""
    _need(k_cache, "k_cache", torch.bfloat16)
    B, H, cap, D = k_cache.shape
    _need(v_cache, "v_cache", torch.bfloat16, (B, H, cap, D))
    _need(q, "q", torch.float32, (B, H, D))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("decode_attn_static_noalloc", lib().dakv_decode_attn_static_noalloc(
        _p(q), _p(k_cache), _p(v_cache), _p(mask), _p(valid_len), B, H, cap, D, float(scale),
        _p(out), _p(lse), int(num_splits), _p(err_flag), _stream()))
    return out, lse


def decode_step_static(q, k_cache, v_cache, k_new, v_new, write_pos, mask=None, valid_len=None,
                       scale=None, out=None, lse=None, workspace=None, num_splits=0,
                       err_flag=None, want_lse=True):
    """kv_append followed by decode_attn_static, in one pass.  Returns ``(out, lse)``."""
    _need(k_cache, "k_cache", torch.bfloat16)
    B, H, cap, D = k_cache.shape
    _need(v_cache, "v_cache", torch.bfloat16, (B, H, cap, D))
    _need(q, "q", torch.float32, (B, H, D))
    _need(k_new, "k_new", torch.bfloat16, (B, H, D))
    _need(v_new, "v_new", torch.bfloat16, (B, H, D))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(mask, "mask", torch.int32, (B, cap))
    _opt(valid_len, "valid_len", torch.int32, (B,))
    if mask is None and valid_len is None:
        raise ValueError("give a mask, a valid length, or both")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, H))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = decode_attn_static_workspace_size(B, H, cap, D)
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_step_static", lib().dakv_decode_step_static(
        _p(q), _p(k_cache), _p(v_cache), _p(k_new), _p(v_new), _p(write_pos), _p(mask),
        _p(valid_len), B, H, cap, D, float(scale), _p(out), _p(lse), _p(ws), ws.numel(),
        int(num_splits), _p(err_flag), _stream()))
    return out, lse


# ---------------------------------------------------------- gather_pa_kv_cache


def gather_pa_kv_cache(key_cache, value_cache, block_tables, seq_lens, seq_offset=None,
                       total_tokens=None, key_out=None, value_out=None, err_flag=None,
                       validate=True):
    """Collect paged K/V rows into contiguous [total_tokens, H, D] outputs (bit copy).

    With ``validate`` the index tensors are copied to the host and checked first
    (the index tensors are host-ready on the pages); ``total_tokens`` defaults to
    seq_lens[Q] read on the host.
    """
    _need(key_cache, "key_cache", torch.bfloat16)
    _need(value_cache, "value_cache", torch.bfloat16)
    if key_cache.dim() != 4 or value_cache.dim() != 4:
        raise ValueError("caches must be [num_blocks, block_size, heads, dim]")
    nb, bs, Hk, Dk = key_cache.shape
    nb2, bs2, Hv, Dv = value_cache.shape
    if (nb, bs) != (nb2, bs2):
        raise ValueError("key_cache and value_cache must agree on num_blocks, block_size")
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [Q, cols]")
    Q, cols = block_tables.shape
    _need(seq_lens, "seq_lens", torch.int32)
    if tuple(seq_lens.shape) != (Q + 1,):
        raise ValueError("only cumulative seq_lens [Q + 1] is supported")
    _opt(seq_offset, "seq_offset", torch.int32, (Q,))
    if validate:
        validate_paged(block_tables, seq_lens, seq_offset, nb, bs)
    if total_tokens is None:
        total_tokens = int(_host_i32(seq_lens)[-1])
    T = int(total_tokens)
    if key_out is None:
        key_out = torch.empty((T, Hk, Dk), dtype=torch.bfloat16, device=key_cache.device)
    if value_out is None:
        value_out = torch.empty((T, Hv, Dv), dtype=torch.bfloat16, device=key_cache.device)
    _need(key_out, "key_out", torch.bfloat16, (T, Hk, Dk))
    _need(value_out, "value_out", torch.bfloat16, (T, Hv, Dv))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("gather_pa_kv_cache", lib().dakv_gather_pa_kv_cache(
        _p(key_cache), _p(value_cache), nb, bs, Hk, Dk, Hv, Dv, _p(block_tables), Q, cols,
        _p(seq_lens), _p(seq_offset), T, _p(key_out), _p(value_out), _p(err_flag), _stream()))
    return key_out, value_out


# ----------------------------------------------------------- decode_attn_paged


def decode_attn_paged_workspace_size(B, Hq, D, max_seq_len, block_size):
    return int(lib().dakv_decode_attn_paged_workspace_size(B, Hq, D, max_seq_len, block_size))


def decode_attn_paged(q, key_cache, value_cache, block_tables, seq_lens, seq_offset=None,
                      max_seq_len=None, scale=None, out=None, lse=None, workspace=None,
                      num_splits=0, err_flag=None, validate=False, want_lse=True):
    """Paged GQA decode attention.  Returns ``(out, lse)``.

    q bf16 [B, Hq, D]; caches bf16 [num_blocks, block_size, Hkv, D]; block_tables
    int32 [B, cols]; cumulative seq_lens int32 [B + 1]; ``max_seq_len`` is a host
    upper bound of the lengths (read from seq_lens on the host when omitted).
    """
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    _need(key_cache, "key_cache", torch.bfloat16)
    nb, bs, Hkv, Dk = key_cache.shape
    if Dk != D:
        raise ValueError("key_cache head dim must equal q's")
    _need(value_cache, "value_cache", torch.bfloat16, (nb, bs, Hkv, D))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, cols]")
    cols = block_tables.shape[1]
    _need(seq_lens, "seq_lens", torch.int32, (B + 1,))
    _opt(seq_offset, "seq_offset", torch.int32, (B,))
    if validate:
        validate_paged(block_tables, seq_lens, seq_offset, nb, bs)
    if max_seq_len is None:
        lens = np.diff(_host_i32(seq_lens))
        max_seq_len = int(lens.max()) if lens.size else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = decode_attn_paged_workspace_size(B, Hq, D, int(max_seq_len), bs)
    ws = _workspace(nbytes, q.device, workspace)
    check("decode_attn_paged", lib().dakv_decode_attn_paged(
        _p(q), _p(key_cache), _p(value_cache), _p(block_tables), cols, _p(seq_lens),
        _p(seq_offset), B, Hq, Hkv, D, nb, bs, int(max_seq_len), float(scale), _p(out), _p(lse),
        _p(ws), ws.numel(), int(num_splits), _p(err_flag), _stream()))
    return out, lse


def _paged_append_lowbit(fmt, k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                         block_tables, seq_lens, seq_offset, err_flag):
    per = 2 if fmt == "fp4" else 1          # values per code byte
    _need(k_codes, "k_codes", torch.uint8)
    nb, bs, Hkv, Dc = k_codes.shape
    D = Dc * per
    _need(v_codes, "v_codes", torch.uint8, (nb, bs, Hkv, Dc))
    _need(k_scale, "k_scale", torch.float32, (nb, bs, Hkv))
    _need(v_scale, "v_scale", torch.float32, (nb, bs, Hkv))
    _need(k_new, "k_new", torch.bfloat16)
    B = k_new.shape[0]
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, D))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, D))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, cols]")
    _need(seq_lens, "seq_lens", torch.int32, (B + 1,))
    _opt(seq_offset, "seq_offset", torch.int32, (B,))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    name = "paged_append_" + fmt
    check(name, getattr(lib(), "dakv_" + name)(
        _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(k_new), _p(v_new),
        _p(block_tables), block_tables.shape[1], _p(seq_lens), _p(seq_offset), B, Hkv, D, nb,
        bs, _p(err_flag), _stream()))


def paged_append_fp8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_tables,
                     seq_lens, seq_offset=None, err_flag=None):
    """Quantise each sequence's new token (bf16 [B, Hkv, D]) into its last position
    len_b - 1 of the FP8 pool (codes uint8 [num_blocks, block_size, Hkv, D], scales
    fp32 [num_blocks, block_size, Hkv]), placed through the block table."""
    _paged_append_lowbit("fp8", k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                         block_tables, seq_lens, seq_offset, err_flag)


def paged_append_fp4(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_tables,
                     seq_lens, seq_offset=None, err_flag=None):
    """As paged_append_fp8 into the FP4 pool (E2M1 codes two per byte, element 2i in
    the low four bits: uint8 [num_blocks, block_size, Hkv, D / 2])."""
    _paged_append_lowbit("fp4", k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                         block_tables, seq_lens, seq_offset, err_flag)


def _decode_attn_paged_lowbit(fmt, q, k_codes, v_codes, k_scale, v_scale, block_tables,
                              seq_lens, seq_offset, max_seq_len, scale, out, lse, workspace,
                              num_splits, err_flag, validate, want_lse):
    per = 2 if fmt == "fp4" else 1          # values per code byte
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    _need(k_codes, "k_codes", torch.uint8)
    nb, bs, Hkv, Dc = k_codes.shape
    if Dc * per != D:
        raise ValueError("the pool's head dim must equal q's")
    _need(v_codes, "v_codes", torch.uint8, (nb, bs, Hkv, Dc))
    _need(k_scale, "k_scale", torch.float32, (nb, bs, Hkv))
    _need(v_scale, "v_scale", torch.float32, (nb, bs, Hkv))
    _need(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, cols]")
    cols = block_tables.shape[1]
    _need(seq_lens, "seq_lens", torch.int32, (B + 1,))
    _opt(seq_offset, "seq_offset", torch.int32, (B,))
    if validate:
        validate_paged(block_tables, seq_lens, seq_offset, nb, bs)
    if max_seq_len is None:
        lens = np.diff(_host_i32(seq_lens))
        max_seq_len = int(lens.max()) if lens.size else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = decode_attn_paged_workspace_size(B, Hq, D, int(max_seq_len), bs)
    ws = _workspace(nbytes, q.device, workspace)
    name = "decode_attn_paged_" + fmt
    check(name, getattr(lib(), "dakv_" + name)(
        _p(q), _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale), _p(block_tables), cols,
        _p(seq_lens), _p(seq_offset), B, Hq, Hkv, D, nb, bs, int(max_seq_len), float(scale),
        _p(out), _p(lse), _p(ws), ws.numel(), int(num_splits), _p(err_flag), _stream()))
    return out, lse


def decode_attn_paged_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens,
                          seq_offset=None, max_seq_len=None, scale=None, out=None, lse=None,
                          workspace=None, num_splits=0, err_flag=None, validate=False,
                          want_lse=True):
    """decode_attn_paged over the FP8 pool.  Returns ``(out, lse)``."""
    return _decode_attn_paged_lowbit("fp8", q, k_codes, v_codes, k_scale, v_scale,
                                     block_tables, seq_lens, seq_offset, max_seq_len, scale,
                                     out, lse, workspace, num_splits, err_flag, validate,
                                     want_lse)


def decode_attn_paged_fp4(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens,
                          seq_offset=None, max_seq_len=None, scale=None, out=None, lse=None,
                          workspace=None, num_splits=0, err_flag=None, validate=False,
                          want_lse=True):
    """decode_attn_paged over the FP4 pool (packed codes uint8 [num_blocks,
    block_size, Hkv, D / 2]).  Returns ``(out, lse)``."""
    return _decode_attn_paged_lowbit("fp4", q, k_codes, v_codes, k_scale, v_scale,
                                     block_tables, seq_lens, seq_offset, max_seq_len, scale,
                                     out, lse, workspace, num_splits, err_flag, validate,
                                     want_lse)


# ----------------------------------------------------- sparse_topk_decode_attn


def sparse_topk_decode_attn_workspace_size(B, Hq, d_qk, d_v, topk):
    return int(lib().dakv_sparse_topk_decode_attn_workspace_size(B, Hq, d_qk, d_v, topk))


def sparse_topk_decode_attn(q, kv, indices, d_v=512, sm_scale=None, out=None, lse=None,
                            workspace=None, err_flag=None, validate=False, want_lse=True):
    """Top-k sparse MLA-style decode.  Returns ``(out, lse)``.

    q bf16 [B, Hq, d_qk]; kv bf16 [B, s_kv, d_qk]; indices int32 [B, topk].
    """
    _need(q, "q", torch.bfloat16)
    B, Hq, d_qk = q.shape
    _need(kv, "kv", torch.bfloat16)
    if kv.dim() != 3 or kv.shape[0] != B or kv.shape[2] != d_qk:
        raise ValueError("kv must be [B, s_kv, d_qk]")
    s_kv = kv.shape[1]
    _need(indices, "indices", torch.int32)
    if indices.dim() != 2 or indices.shape[0] != B:
        raise ValueError("indices must be [B, topk]")
    topk = indices.shape[1]
    if validate:
        validate_sparse(indices, s_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((B, Hq, d_v), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, d_v))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = sparse_topk_decode_attn_workspace_size(B, Hq, d_qk, d_v, topk)
    ws = _workspace(nbytes, q.device, workspace)
    check("sparse_topk_decode_attn", lib().dakv_sparse_topk_decode_attn(
        _p(q), _p(kv), _p(indices), B, Hq, s_kv, d_qk, d_v, topk, float(sm_scale), _p(out),
        _p(lse), _p(ws), ws.numel(), _p(err_flag), _stream()))
    return out, lse


def sparse_topk_attn(q, kv, indices, d_v=512, sm_scale=None, out=None, lse=None,
                     workspace=None, err_flag=None, validate=False, want_lse=True):
    """Top-k sparse MLA-style attention with several q-tokens per sequence, each with
    its own index list into the sequence's latent cache.  Returns ``(out, lse)``.

    q bf16 [B, s_q, Hq, d_qk]; kv bf16 [B, s_kv, d_qk]; indices int32 [B, s_q, topk];
    out fp32 [B, s_q, Hq, d_v]; lse fp32 [B, s_q, Hq].
    """
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, s_q, Hq, d_qk]")
    B, s_q, Hq, d_qk = q.shape
    _need(kv, "kv", torch.bfloat16)
    if kv.dim() != 3 or kv.shape[0] != B or kv.shape[2] != d_qk:
        raise ValueError("kv must be [B, s_kv, d_qk]")
    s_kv = kv.shape[1]
    _need(indices, "indices", torch.int32)
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    topk = indices.shape[2]
    if validate:
        validate_sparse(indices.reshape(B * s_q, topk), s_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((B, s_q, Hq, d_v), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, s_q, Hq, d_v))
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, s_q, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = sparse_topk_decode_attn_workspace_size(B * s_q, Hq, d_qk, d_v, topk)
    ws = _workspace(nbytes, q.device, workspace)
    check("sparse_topk_attn", lib().dakv_sparse_topk_attn(
        _p(q), _p(kv), _p(indices), B, s_q, Hq, s_kv, d_qk, d_v, topk, float(sm_scale),
        _p(out), _p(lse), _p(ws), ws.numel(), _p(err_flag), _stream()))
    return out, lse


def latent_append_fp8(codes, scale, new_rows, write_pos, err_flag=None):
    """Quantise each sequence's new latent row (bf16 [B, d_qk]) to E4M3 codes with a
    power-of-two scale and store them at row write_pos[b] of codes uint8
    [B, s_kv, d_qk] and scale fp32 [B, s_kv]."""
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3:
        raise ValueError("codes must be [B, s_kv, d_qk]")
    B, s_kv, d_qk = codes.shape
    _need(scale, "scale", torch.float32, (B, s_kv))
    _need(new_rows, "new_rows", torch.bfloat16, (B, d_qk))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("latent_append_fp8", lib().dakv_latent_append_fp8(
        _p(codes), _p(scale), _p(new_rows), _p(write_pos), B, s_kv, d_qk, _p(err_flag),
        _stream()))


def sparse_topk_attn_fp8(q, codes, scale, indices, d_v=512, sm_scale=None, out=None, lse=None,
                         workspace=None, err_flag=None, validate=False, want_lse=True):
    """sparse_topk_attn over the FP8 latent cache (codes uint8 [B, s_kv, d_qk], scale
    fp32 [B, s_kv]).  q bf16 [B, s_q, Hq, d_qk]; indices int32 [B, s_q, topk].
    Returns ``(out, lse)``."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, s_q, Hq, d_qk]")
    B, s_q, Hq, d_qk = q.shape
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3 or codes.shape[0] != B or codes.shape[2] != d_qk:
        raise ValueError("codes must be [B, s_kv, d_qk]")
    s_kv = codes.shape[1]
    _need(scale, "scale", torch.float32, (B, s_kv))
    _need(indices, "indices", torch.int32)
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    topk = indices.shape[2]
    if validate:
        validate_sparse(indices.reshape(B * s_q, topk), s_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((B, s_q, Hq, d_v), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, s_q, Hq, d_v))
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, s_q, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = sparse_topk_decode_attn_workspace_size(B * s_q, Hq, d_qk, d_v, topk)
    ws = _workspace(nbytes, q.device, workspace)
    check("sparse_topk_attn_fp8", lib().dakv_sparse_topk_attn_fp8(
        _p(q), _p(codes), _p(scale), _p(indices), B, s_q, Hq, s_kv, d_qk, d_v, topk,
        float(sm_scale), _p(out), _p(lse), _p(ws), ws.numel(), _p(err_flag), _stream()))
    return out, lse


def latent_append_fp4(codes, scale, new_rows, write_pos, err_flag=None):
    """Quantise each sequence's new latent row (bf16 [B, d_qk]) to E2M1 codes (two per
    byte, element 2i in the low four bits) with a power-of-two scale and store them at
    row write_pos[b] of codes uint8 [B, s_kv, d_qk / 2] and scale fp32 [B, s_kv]."""
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3:
        raise ValueError("codes must be [B, s_kv, d_qk / 2]")
    B, s_kv, half = codes.shape
    d_qk = 2 * half
    _need(scale, "scale", torch.float32, (B, s_kv))
    _need(new_rows, "new_rows", torch.bfloat16, (B, d_qk))
    _need(write_pos, "write_pos", torch.int32, (B,))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    check("latent_append_fp4", lib().dakv_latent_append_fp4(
        _p(codes), _p(scale), _p(new_rows), _p(write_pos), B, s_kv, d_qk, _p(err_flag),
        _stream()))


def sparse_topk_attn_fp4(q, codes, scale, indices, d_v=512, sm_scale=None, out=None, lse=None,
                         workspace=None, err_flag=None, validate=False, want_lse=True):
    """sparse_topk_attn over the FP4 latent cache (codes uint8 [B, s_kv, d_qk / 2],
    scale fp32 [B, s_kv]).  q bf16 [B, s_q, Hq, d_qk]; indices int32 [B, s_q, topk].
    Returns ``(out, lse)``."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, s_q, Hq, d_qk]")
    B, s_q, Hq, d_qk = q.shape
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3 or codes.shape[0] != B or 2 * codes.shape[2] != d_qk:
        raise ValueError("codes must be [B, s_kv, d_qk / 2]")
    s_kv = codes.shape[1]
    _need(scale, "scale", torch.float32, (B, s_kv))
    _need(indices, "indices", torch.int32)
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    topk = indices.shape[2]
    if validate:
        validate_sparse(indices.reshape(B * s_q, topk), s_kv)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((B, s_q, Hq, d_v), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, s_q, Hq, d_v))
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, Hq), dtype=torch.float32, device=q.device)
    _opt(lse, "lse", torch.float32, (B, s_q, Hq))
    _opt(err_flag, "err_flag", torch.int32, (1,))
    nbytes = sparse_topk_decode_attn_workspace_size(B * s_q, Hq, d_qk, d_v, topk)
    ws = _workspace(nbytes, q.device, workspace)
    check("sparse_topk_attn_fp4", lib().dakv_sparse_topk_attn_fp4(
        _p(q), _p(codes), _p(scale), _p(indices), B, s_q, Hq, s_kv, d_qk, d_v, topk,
        float(sm_scale), _p(out), _p(lse), _p(ws), ws.numel(), _p(err_flag), _stream()))
    return out, lse
