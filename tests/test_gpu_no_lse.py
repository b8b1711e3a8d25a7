"""GPU: calls that ask for no log-sum-exp (the library gets a null lse pointer) write the
same outputs, bit for bit, as calls that do -- through a direct single-split output and
through each kind of split merge."""

import numpy as np
import pytest
import torch

import workloads
import decode_attention_kv_amd as dakv
from conftest import npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def same_without_lse(call):
    out_a, lse_a = call(True)
    out_b, lse_b = call(False)
    torch.cuda.synchronize()
    assert lse_a is not None and lse_b is None
    assert np.array_equal(npy(out_a), npy(out_b))


@pytest.mark.parametrize("lengths", [[5000, 0, 1, 3000, 17], [300, 17]])
def test_paged_without_lse(lengths):
    """Matrix-core kernel: pieces merged (first), whole groups written directly (second)."""
    case = workloads.paged_case(lengths, Hq=32, Hkv=8, D=128, block_size=16, device=DEV,
                                seed=190)
    t = torch.from_numpy(case.index.block_tables).to(DEV)
    s = torch.from_numpy(case.index.seq_lens).to(DEV)
    o = None if case.index.seq_offset is None else torch.from_numpy(case.index.seq_offset).to(DEV)
    same_without_lse(lambda w: dakv.decode_attn_paged(case.q, case.key_cache, case.value_cache,
                                                      t, s, o, scale=case.scale, want_lse=w))


@pytest.mark.parametrize("num_splits", [0, 1])
def test_static_without_lse(num_splits):
    case = workloads.static_case(3, 8, 128, 4096, [4000, 1, 2600], device=DEV, seed=191)
    same_without_lse(lambda w: dakv.decode_attn_static(
        case.q, case.k_cache, case.v_cache, mask=case.mask, valid_len=case.valid_len,
        scale=case.scale, num_splits=num_splits, want_lse=w))


def test_sparse_without_lse():
    case = workloads.sparse_case(2, 64, 5000, 1500, device=DEV, seed=192)
    same_without_lse(lambda w: dakv.sparse_topk_decode_attn(
        case.q, case.kv, case.indices, d_v=case.d_v, sm_scale=case.sm_scale, want_lse=w))
