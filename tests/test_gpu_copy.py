"""GPU parity: the prefill -> generate KV copy and the mask roll-back, bit-exact
against the fp64 oracle (copies move 16-bit patterns untouched)."""

import numpy as np
import pytest
import torch

import oracle
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, bits, npy


def raw16(t):
    """The 16-bit patterns of a bf16 or fp16 tensor, on the CPU."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_tensor(g, shape, std=1.0, dtype=torch.bfloat16):
    return (torch.randn(shape, generator=g, device=DEV) * std).to(dtype)


def make(n, B, H, S_src, S_dst, D, seed, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    src = [bf16_tensor(g, (B, H, S_src, D), dtype=dtype) for _ in range(n)]
    dst = [bf16_tensor(g, (B, H, S_dst, D), std=100.0, dtype=dtype) for _ in range(n)]
    return src, dst


def check_copy(src, dst, lengths, with_mask=True, flag=None):
    B = src[0].shape[0]
    S_dst = dst[0].shape[2]
    before = [raw16(d) for d in dst]
    lens = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    mask = torch.full((B, S_dst), 7, dtype=torch.int32, device=DEV) if with_mask else None
    dakv.copy_kvcache(src, dst, lens, mask=mask, err_flag=flag)
    torch.cuda.synchronize()
    lim = min(src[0].shape[2], S_dst)
    clamped = [min(max(n, 0), lim) for n in lengths]
    want, want_mask = oracle.copy_kvcache([raw16(s) for s in src], before, clamped,
                                          None if mask is None else np.zeros((B, S_dst), np.int32))
    for d, w in zip(dst, want):
        assert np.array_equal(raw16(d), w)
    if with_mask:
        assert np.array_equal(npy(mask), want_mask)


def test_copy_prompt_rows_ragged_bit_exact():
    """Prefill capacity 1024, generate 1152; prompts of 4 (the page's example), 1024
    and 0 rows; two layers' K and V."""
    src, dst = make(4, 3, 4, 1024, 1152, 128, seed=1)
    check_copy(src, dst, [4, 1024, 0])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_copy_head_dim_64_and_smaller_destination(dtype):
    src, dst = make(3, 2, 2, 40, 33, 64, seed=2, dtype=dtype)
    check_copy(src, dst, [33, 17])


def test_copy_length_outside_the_buffers_is_clamped_and_flagged():
    src, dst = make(2, 2, 2, 64, 80, 128, seed=3)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    check_copy(src, dst, [2000, -3], flag=flag)
    assert int(flag.item()) & dakv._lib.ERR_COPY_LEN


def test_copy_7b_hand_over_sampled():
    """The page's 7B hand-over: 32 layers x K and V = 64 tensors [1, 32, 1024 -> 1152,
    128], 1024 rows each (512 MiB); four of the 64 compared with the oracle, and every
    tensor's copied and kept rows checked on the device."""
    print("copy_kvcache 64 tensors", flush=True)
    src, dst = make(64, 1, 32, 1024, 1152, 128, seed=4)
    keep = [d[:, :, 1024:].clone() for d in dst]
    sample = [0, 17, 40, 63]
    before = [bits(dst[i]) for i in sample]
    lens = torch.tensor([1024], dtype=torch.int32, device=DEV)
    dakv.copy_kvcache(src, dst, lens)
    torch.cuda.synchronize()
    for i in range(64):
        assert torch.equal(dst[i][:, :, :1024].view(torch.int16), src[i].view(torch.int16))
        assert torch.equal(dst[i][:, :, 1024:].view(torch.int16), keep[i].view(torch.int16))
    want, _ = oracle.copy_kvcache([bits(src[i]) for i in sample], before, [1024])
    for j, i in enumerate(sample):
        assert np.array_equal(bits(dst[i]), want[j])


def test_trim_matches_oracle_and_flags_bad_lengths():
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    mask = (torch.rand((4, 300), generator=g, device=DEV) > 0.3).to(torch.int32)
    before = npy(mask)
    new_len = torch.tensor([150, 0, 300, 7], dtype=torch.int32, device=DEV)
    dakv.trim_kvcache(mask, new_len)
    torch.cuda.synchronize()
    assert np.array_equal(npy(mask), oracle.trim_kvcache(before, [150, 0, 300, 7]))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.trim_kvcache(mask, torch.tensor([400, -1, 5, 5], dtype=torch.int32, device=DEV),
                      err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_COPY_LEN
    assert np.array_equal(npy(mask), oracle.trim_kvcache(oracle.trim_kvcache(before, [150, 0, 300, 7]),
                                                         [300, 0, 5, 5]))


def test_copy_then_decode_attends_exactly_the_prompt():
    """End to end: hand-over, then the generate model's masked decode attention equals
    the oracle's attention over the prefill rows."""
    src, dst = make(2, 2, 4, 256, 320, 128, seed=6)
    lengths = [100, 256]
    lens = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    mask = torch.ones((2, 320), dtype=torch.int32, device=DEV)
    dakv.copy_kvcache(src, dst, lens, mask=mask)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    q = torch.randn((2, 4, 128), generator=g, device=DEV)
    out, _ = dakv.decode_attn_static(q, dst[0], dst[1], mask=mask)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_static(npy(q), bits(src[0]), bits(src[1]), valid_len=lengths)
    assert_attention_close(npy(out), ref)
