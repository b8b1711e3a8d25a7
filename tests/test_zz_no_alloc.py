"""GPU: dakv_decode_attn_static_noalloc (split partials in the library's fixed device
scratch, no workspace argument) against dakv_decode_attn_static (caller workspace) on
the same inputs, through the C-ABI: two calls in a row, the second smaller, each bit
for bit equal to the workspace entry point and within the attention tolerance of the
oracle on sampled sequences.  The scratch keeps the previous call's contents, so the
second call also shows that nothing is read from it before it is written."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def both(case, num_splits=0):
    out_ws, lse_ws = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache,
                                             mask=case.mask, valid_len=case.valid_len,
                                             scale=case.scale, num_splits=num_splits)
    out_na, lse_na = dakv.decode_attn_static_noalloc(case.q, case.k_cache, case.v_cache,
                                                     mask=case.mask, valid_len=case.valid_len,
                                                     scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return npy(out_ws), npy(lse_ws), npy(out_na), npy(lse_na)


def check_against_oracle(case, out, lse, seqs):
    for b in seqs:
        L = case.lengths[b]
        ref_out, ref_lse = oracle.decode_static(npy(case.q[b:b + 1]),
                                                bits(case.k_cache[b:b + 1, :, :L]),
                                                bits(case.v_cache[b:b + 1, :, :L]),
                                                npy(case.mask[b:b + 1, :L]), [L], case.scale)
        assert_attention_close(out[b:b + 1], ref_out)
        assert_lse_close(lse[b:b + 1], ref_lse)


def test_noalloc_matches_workspace_entry_on_two_calls_second_smaller():
    # call 1: the 7B-shaped layer at batch 8 (128-row splits, 4.2 MB of partials)
    lengths = workloads.uniform_lengths(8, 1, 4096, 2)
    print(f"noalloc call 1: B=8 H=32 D=128 cap=4096 lengths={lengths}", flush=True)
    need = dakv.lib().dakv_decode_attn_static_noalloc_scratch_bytes(8, 32, 4096, 128, 0)
    assert 0 < need <= dakv._lib.NOALLOC_SCRATCH_BYTES
    big = workloads.static_case(8, 32, 128, 4096, lengths, device=DEV, seed=51,
                                mask_density=0.9)
    o_ws, l_ws, o_na, l_na = both(big)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)
    check_against_oracle(big, o_na, l_na, [0, int(np.argmax(lengths)), 7])
    del big
    # call 2: smaller (head_dim 64, 64-row splits), scratch still holding call 1's data
    print("noalloc call 2: B=2 H=4 D=64 cap=1152", flush=True)
    small = workloads.static_case(2, 4, 64, 1152, [1152, 103], device=DEV, seed=52)
    o_ws, l_ws, o_na, l_na = both(small)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)
    check_against_oracle(small, o_na, l_na, [0, 1])
    # forced split counts share the same scratch
    o_ws, l_ws, o_na, l_na = both(small, num_splits=7)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)


def test_noalloc_rejects_calls_beyond_the_scratch():
    B, H, cap, D = 64, 32, 4096, 128
    assert dakv.lib().dakv_decode_attn_static_noalloc_scratch_bytes(B, H, cap, D, 0) > \
        dakv._lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, D), device=DEV)
    kv = torch.zeros((B, H, cap, D), dtype=torch.bfloat16, device=DEV)
    vl = torch.ones(B, dtype=torch.int32, device=DEV)
    with pytest.raises(dakv.DakvError) as e:
        dakv.decode_attn_static_noalloc(q, kv, kv, valid_len=vl)
    assert e.value.code == dakv._lib.ESCRATCH
