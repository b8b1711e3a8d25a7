"""ctypes loader of libdakv.so: the C-ABI declared in include/dakv.h.

The library is built in-tree (``python -m decode_attention_kv_amd.build``).  There is
no fallback: if the shared library is missing, loading fails loudly.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdakv.so")

OK = 0
EINVAL = -1
ENOTSUP = -2
ERANGE = -3
EHIP = -4
ESCRATCH = -5
NOALLOC_SCRATCH_BYTES = 16 << 20

ERR_BLOCK_ID = 1
ERR_WRITE_POS = 2
ERR_SPARSE_INDEX = 4
ERR_SEQ_LENS = 8
ERR_VALID_LEN = 16
ERR_COPY_LEN = 32
COPY_MAX_TENSORS = 128

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/dakv.h
SIGNATURES = {
    "dakv_strerror": (ctypes.c_char_p, [_i]),
    "dakv_kv_append": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "dakv_kv_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp,
                                _vp]),
    "dakv_decode_attn_static_fp8_workspace_size": (_sz, [_i, _i, _i, _i]),
    "dakv_decode_attn_static_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                                         _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_kv_append_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp,
                                _vp]),
    "dakv_decode_attn_static_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                                         _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_decode_step_static_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                         _i, _i, _i, _f, _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_decode_step_static_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                         _i, _i, _i, _f, _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_copy_kvcache": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "dakv_trim_kvcache": (_i, [_vp, _vp, _i, _i, _vp, _vp]),
    "dakv_decode_attn_static_workspace_size": (_sz, [_i, _i, _i, _i]),
    "dakv_decode_attn_static_split_rows": (_i, [_i, _i, _i, _i, _i]),
    "dakv_decode_attn_static_noalloc_scratch_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dakv_decode_attn_static_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp,
                                             _vp, _i, _vp, _vp]),
    "dakv_decode_attn_static": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _vp,
                                     _vp, _sz, _i, _vp, _vp]),
    "dakv_decode_step_static": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                                     _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_gather_pa_kv_cache": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp,
                                     _i, _vp, _vp, _vp, _vp]),
    "dakv_decode_attn_paged_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "dakv_decode_attn_paged": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                    _i, _f, _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    "dakv_sparse_topk_decode_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "dakv_sparse_topk_decode_attn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                          _vp, _sz, _vp, _vp]),
    "dakv_sparse_topk_attn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                   _vp, _sz, _vp, _vp]),
    "dakv_latent_append_fp8": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "dakv_sparse_topk_attn_fp8": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                       _vp, _vp, _sz, _vp, _vp]),
    "dakv_latent_append_fp4": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "dakv_sparse_topk_attn_fp4": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                       _vp, _vp, _sz, _vp, _vp]),
    "dakv_paged_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i,
                                   _i, _i, _vp, _vp]),
    "dakv_decode_attn_paged_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i,
                                        _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _i, _vp,
                                        _vp]),
    "dakv_paged_append_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i,
                                   _i, _i, _vp, _vp]),
    "dakv_decode_attn_paged_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i,
                                        _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _i, _vp,
                                        _vp]),
    "dakv_validate_paged": (_i, [_vp, _i, _i, _vp, _vp, _i, _i]),
    "dakv_validate_sparse": (_i, [_vp, _i, _i, _i]),
    "dakv_validate_range": (_i, [_vp, _i, _i, _i]),
}

_lib = None


def lib():
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_kv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code):
    return lib().dakv_strerror(int(code)).decode()


class DakvError(ValueError):
    """A nonzero status from the C-ABI."""

    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn}: {strerror(code)} (status {code})")


def check(fn, code):
    if code != OK:
        raise DakvError(fn, code)
