"""Seeded synthetic inputs for decode attention over a KV cache.

This module is shared by the tests, the smoke check and the benchmark; it feeds
both the HIP path and the fp64 oracle and holds none of the method's arithmetic:
only random values, lengths, permutations and table layouts.  Structure (lengths,
block tables, sparse indices) is drawn with ``numpy.random.default_rng(seed)``;
bulk values are drawn with a ``torch.Generator`` on the target device (the oracle
always reads back the exact bf16 bits that were produced, so the generator's
device never affects parity).

Workload recipes (sizes from the decode-attention configurations this library is
measured on):

* ``static_tiny``   -- batch 1, 4 heads, head_dim 64, capacity 1152 = 1024 + 128;
  K/V N(0,1) in the first L rows and N(0, 10^2) garbage after them; fp32 query;
  mask = first L ones; L in {4, 5, 103, 1152}.
* ``static_llama_layer`` -- batch 1 or 8, 32 heads, head_dim 128, capacity 4096,
  32 layers each with its own K/V N(0,1) bf16 cache; L_b uniform on {1..4096},
  the same in every layer; the new token is appended at row L_b - 1 and the mask
  has L_b ones after the append.
* ``gather_nd``     -- key/value cache [8192, 128, 8, 128] bf16 N(0,1); 32
  sequences with lengths uniform on {1..4096}; block tables [32, 64] filled with
  the first 2048 ids of a permutation of the 8192 blocks; seq_offset = 128 * u
  with u uniform on {0 .. 64 - ceil(len/128)}.
* ``paged_gqa``     -- batch 64, 32 query / 8 KV heads, head_dim 128, block 16;
  context lengths log-uniform on [512, 16384]; a pool of
  ceil(1.1 * sum ceil(ctx/16)) blocks; each sequence's blocks take successive ids
  of one random permutation; unused table entries are -1.
* ``sparse_mla``    -- batch 16, 128 query heads on one latent KV per token,
  d_qk = 576, d_v = 512, context 32768, 2048 distinct indices per sequence.
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, gen, device, std=1.0):
    return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


# --------------------------------------------------------------------------- static


@dataclass
class StaticCase:
    q: torch.Tensor               # fp32 [B, H, D]
    k_cache: torch.Tensor         # bf16 [B, H, cap, D]
    v_cache: torch.Tensor         # bf16 [B, H, cap, D]
    mask: Optional[torch.Tensor]  # int32 [B, cap]
    valid_len: Optional[torch.Tensor]  # int32 [B]
    lengths: list                 # host copy of the valid lengths
    scale: float


def static_case(B, H, D, cap, lengths, *, device="cpu", seed=0, garbage_std=10.0,
                with_mask=True, with_valid_len=True, mask_density=1.0):
    """One static-buffer decode problem.

    Rows below L_b hold N(0,1) bf16 values, rows at and above L_b hold N(0, std^2)
    garbage.  ``mask_density < 1`` zeroes a random share of the first L_b mask
    entries (holes inside the valid range).
    """
    lengths = [int(x) for x in lengths]
    assert len(lengths) == B and all(0 <= x <= cap for x in lengths)
    rng = np.random.default_rng(seed)
    g = _gen(device, seed)
    k = _randn_bf16((B, H, cap, D), g, device)
    v = _randn_bf16((B, H, cap, D), g, device)
    rows = torch.arange(cap, device=device)
    for b, L in enumerate(lengths):
        if L < cap:
            k[b, :, L:, :] = _randn_bf16((H, cap - L, D), g, device, garbage_std)
            v[b, :, L:, :] = _randn_bf16((H, cap - L, D), g, device, garbage_std)
    q = torch.randn((B, H, D), generator=g, device=device, dtype=torch.float32)
    mask = None
    if with_mask:
        m = np.zeros((B, cap), dtype=np.int32)
        for b, L in enumerate(lengths):
            m[b, :L] = 1
            if mask_density < 1.0:
                holes = rng.random(L) >= mask_density
                m[b, :L][holes] = 0
        mask = torch.from_numpy(m).to(device)
    valid = torch.tensor(lengths, dtype=torch.int32, device=device) if with_valid_len else None
    del rows
    return StaticCase(q=q, k_cache=k, v_cache=v, mask=mask, valid_len=valid,
                      lengths=lengths, scale=1.0 / math.sqrt(D))


def static_tiny(L, *, device="cpu", seed=1):
    """Batch 1, 4 heads, head_dim 64, capacity 1152, valid length L."""
    return static_case(1, 4, 64, 1152, [L], device=device, seed=seed, garbage_std=10.0)


def uniform_lengths(B, lo, hi, seed):
    """B integers uniform on {lo..hi} (inclusive)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=B)]


@dataclass
class StaticLayer:
    q: torch.Tensor        # fp32 [B, H, D]
    k_cache: torch.Tensor  # bf16 [B, H, cap, D]
    v_cache: torch.Tensor
    k_new: torch.Tensor    # bf16 [B, H, D]
    v_new: torch.Tensor


@dataclass
class StaticModel:
    layers: list
    mask: torch.Tensor       # int32 [B, cap]: first L_b - 1 ones (the append adds row L_b - 1)
    write_pos: torch.Tensor  # int32 [B] = L_b - 1
    valid_len: torch.Tensor  # int32 [B] = L_b
    lengths: list
    B: int
    H: int
    D: int
    cap: int
    scale: float


def static_llama_layers(B, *, n_layers=32, H=32, D=128, cap=4096, device="cpu", seed=2,
                        lengths=None):
    """LLaMA-7B-shaped static decode step: ``n_layers`` independent caches."""
    if lengths is None:
        lengths = uniform_lengths(B, 1, cap, seed)
    g = _gen(device, seed)
    layers = []
    for _ in range(n_layers):
        layers.append(StaticLayer(
            q=torch.randn((B, H, D), generator=g, device=device, dtype=torch.float32),
            k_cache=_randn_bf16((B, H, cap, D), g, device),
            v_cache=_randn_bf16((B, H, cap, D), g, device),
            k_new=_randn_bf16((B, H, D), g, device),
            v_new=_randn_bf16((B, H, D), g, device),
        ))
    m = np.zeros((B, cap), dtype=np.int32)
    for b, L in enumerate(lengths):
        m[b, :L - 1] = 1
    return StaticModel(
        layers=layers,
        mask=torch.from_numpy(m).to(device),
        write_pos=torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device=device),
        valid_len=torch.tensor(lengths, dtype=torch.int32, device=device),
        lengths=list(lengths), B=B, H=H, D=D, cap=cap, scale=1.0 / math.sqrt(D))


# ---------------------------------------------------------------------------- paged


@dataclass
class PagedIndex:
    block_tables: np.ndarray   # int32 [Q, cols]
    seq_lens: np.ndarray       # int32 [Q + 1] cumulative, starting at 0
    seq_offset: Optional[np.ndarray]  # int32 [Q] or None
    lengths: list
    num_blocks: int
    block_size: int


def gather_index(lengths, *, num_blocks, block_size, cols, seed, with_offset=True):
    """Block tables filled with distinct valid ids; random block-aligned offsets.

    The whole table holds the first Q*cols ids of a random permutation of the
    pool, so every entry is valid and distinct; sequence q starts at column
    seq_offset[q] / block_size, drawn so that its used columns fit in the table.
    """
    rng = np.random.default_rng(seed)
    Q = len(lengths)
    assert Q * cols <= num_blocks
    perm = rng.permutation(num_blocks)[: Q * cols].astype(np.int32)
    tables = perm.reshape(Q, cols)
    offs = np.zeros(Q, dtype=np.int32)
    for q, L in enumerate(lengths):
        used = -(-L // block_size)
        assert used <= cols
        if with_offset:
            offs[q] = block_size * int(rng.integers(0, cols - used + 1))
    seq_lens = np.zeros(Q + 1, dtype=np.int32)
    seq_lens[1:] = np.cumsum(lengths)
    return PagedIndex(tables, seq_lens, offs if with_offset else None, list(lengths),
                      num_blocks, block_size)


def pool_index(lengths, *, block_size, slack=0.10, seed):
    """Each sequence's blocks take successive ids of one permutation of the pool.

    The pool holds ceil((1 + slack) * sum ceil(len/block_size)) blocks; the table
    has as many columns as the longest sequence needs; unused entries are -1.
    """
    rng = np.random.default_rng(seed)
    need = [-(-L // block_size) for L in lengths]
    num_blocks = max(1, int(math.ceil((1.0 + slack) * sum(need))))
    cols = max(1, max(need) if need else 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(lengths), cols), -1, dtype=np.int32)
    at = 0
    for q, n in enumerate(need):
        tables[q, :n] = perm[at:at + n]
        at += n
    seq_lens = np.zeros(len(lengths) + 1, dtype=np.int32)
    seq_lens[1:] = np.cumsum(lengths)
    return PagedIndex(tables, seq_lens, None, list(lengths), num_blocks, block_size)


def log_uniform_lengths(B, lo, hi, seed):
    """round(exp(U(ln lo, ln hi))) clipped to [lo, hi]."""
    rng = np.random.default_rng(seed)
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))
    return [int(v) for v in np.clip(np.round(x), lo, hi)]


def paged_caches(num_blocks, block_size, Hk, Dk, Hv, Dv, *, device, seed):
    g = _gen(device, seed)
    return (_randn_bf16((num_blocks, block_size, Hk, Dk), g, device),
            _randn_bf16((num_blocks, block_size, Hv, Dv), g, device))


@dataclass
class GatherCase:
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    index: PagedIndex


def gather_case(lengths, *, num_blocks, block_size, Hk, Dk, Hv, Dv, cols, device="cpu",
                seed=3, with_offset=True):
    index = gather_index(lengths, num_blocks=num_blocks, block_size=block_size, cols=cols,
                         seed=seed, with_offset=with_offset)
    kc, vc = paged_caches(num_blocks, block_size, Hk, Dk, Hv, Dv, device=device, seed=seed)
    return GatherCase(kc, vc, index)


def gather_nd(*, device="cpu", seed=3):
    """Key/value cache [8192, 128, 8, 128], 32 sequences of U{1..4096} tokens."""
    lengths = uniform_lengths(32, 1, 4096, seed)
    return gather_case(lengths, num_blocks=8192, block_size=128, Hk=8, Dk=128, Hv=8, Dv=128,
                       cols=64, device=device, seed=seed)


@dataclass
class PagedCase:
    q: torch.Tensor            # bf16 [B, Hq, D]
    key_cache: torch.Tensor    # bf16 [num_blocks, bs, Hkv, D]
    value_cache: torch.Tensor
    index: PagedIndex
    Hq: int
    Hkv: int
    D: int
    scale: float


def paged_case(lengths, *, Hq, Hkv, D, block_size, device="cpu", seed=4, slack=0.10):
    index = pool_index(lengths, block_size=block_size, slack=slack, seed=seed)
    kc, vc = paged_caches(index.num_blocks, block_size, Hkv, D, Hkv, D, device=device, seed=seed)
    g = _gen(device, seed + 7919)
    q = _randn_bf16((len(lengths), Hq, D), g, device)
    return PagedCase(q, kc, vc, index, Hq, Hkv, D, 1.0 / math.sqrt(D))


def paged_gqa(*, device="cpu", seed=4):
    """Batch 64, 32/8 heads, head_dim 128, block 16, context log-uniform [512, 16384]."""
    lengths = log_uniform_lengths(64, 512, 16384, seed)
    return paged_case(lengths, Hq=32, Hkv=8, D=128, block_size=16, device=device, seed=seed)


# --------------------------------------------------------------------------- sparse


@dataclass
class SparseCase:
    q: torch.Tensor        # bf16 [B, Hq, d_qk]
    kv: torch.Tensor       # bf16 [B, s_kv, d_qk]
    indices: torch.Tensor  # int32 [B, topk]
    d_v: int
    sm_scale: float


def sparse_case(B, Hq, s_kv, topk, *, d_qk=576, d_v=512, device="cpu", seed=5,
                sm_scale=None):
    """Distinct indices per sequence, drawn without replacement."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(B)]).astype(np.int32)
    g = _gen(device, seed)
    kv = _randn_bf16((B, s_kv, d_qk), g, device)
    q = _randn_bf16((B, Hq, d_qk), g, device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    return SparseCase(q, kv, torch.from_numpy(idx).to(device), d_v, float(sm_scale))


def sparse_tokens_case(B, s_q, Hq, s_kv, topk, *, d_qk=576, d_v=512, device="cpu", seed=6,
                       sm_scale=None):
    """Several q-tokens per sequence: q [B, s_q, Hq, d_qk], one latent cache
    kv [B, s_kv, d_qk] per sequence, indices [B, s_q, topk] distinct within a token
    (each token draws its own list without replacement)."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(s_q)])
                    for _ in range(B)]).astype(np.int32).reshape(B, s_q, topk)
    g = _gen(device, seed)
    kv = _randn_bf16((B, s_kv, d_qk), g, device)
    q = _randn_bf16((B, s_q, Hq, d_qk), g, device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    return SparseCase(q, kv, torch.from_numpy(idx).to(device), d_v, float(sm_scale))


@dataclass
class SparseFp8Case:
    q: torch.Tensor        # bf16 [B, s_q, Hq, d_qk]
    codes: torch.Tensor    # uint8 [B, s_kv, d_qk], E4M3 codes (no NaN code)
    scale: torch.Tensor    # fp32 [B, s_kv], powers of two
    indices: torch.Tensor  # int32 [B, s_q, topk]
    d_v: int
    sm_scale: float


def sparse_fp8_case(B, s_q, Hq, s_kv, topk, *, d_qk=576, d_v=512, device="cpu", seed=7,
                    sm_scale=None):
    """An FP8 latent cache as stored bytes: uniformly drawn finite E4M3 codes (the two
    NaN codes are replaced by 0x7E) and row scales 2^-12 .. 2^-6, so the cached values
    reach about 7 in magnitude, as those of quantised O(1) rows do; q bf16 N(0,1);
    indices distinct within a token."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(s_q)])
                    for _ in range(B)]).astype(np.int32).reshape(B, s_q, topk)
    g = _gen(device, seed)
    codes = torch.randint(0, 256, (B, s_kv, d_qk), generator=g, device=device,
                          dtype=torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    e = torch.randint(-12, -5, (B, s_kv), generator=g, device=device, dtype=torch.int32)
    scale = torch.exp2(e.to(torch.float32))
    q = _randn_bf16((B, s_q, Hq, d_qk), g, device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    return SparseFp8Case(q, codes, scale, torch.from_numpy(idx).to(device), d_v,
                         float(sm_scale))


def sparse_fp4_case(B, s_q, Hq, s_kv, topk, *, d_qk=576, d_v=512, device="cpu", seed=8,
                    sm_scale=None):
    """An FP4 latent cache as stored bytes: uniformly drawn bytes (two E2M1 codes each,
    every code finite) ``[B, s_kv, d_qk / 2]`` and row scales 2^-3 .. 2^0, so the cached
    values reach 6 in magnitude; q bf16 N(0,1); indices distinct within a token.
    Returned in a SparseFp8Case (codes packed)."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(s_q)])
                    for _ in range(B)]).astype(np.int32).reshape(B, s_q, topk)
    g = _gen(device, seed)
    codes = torch.randint(0, 256, (B, s_kv, d_qk // 2), generator=g, device=device,
                          dtype=torch.uint8)
    e = torch.randint(-3, 1, (B, s_kv), generator=g, device=device, dtype=torch.int32)
    scale = torch.exp2(e.to(torch.float32))
    q = _randn_bf16((B, s_q, Hq, d_qk), g, device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    return SparseFp8Case(q, codes, scale, torch.from_numpy(idx).to(device), d_v,
                         float(sm_scale))


def sparse_mla(*, device="cpu", seed=5):
    """Batch 16, 128 heads, d_qk 576 / d_v 512, context 32768, top-2048."""
    return sparse_case(16, 128, 32768, 2048, device=device, seed=seed)
