"""GPU parity: kv_append and decode_attn_static (HIP, through the C-ABI) vs the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_static(case, **kw):
    out, lse = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache, mask=case.mask,
                                       valid_len=case.valid_len, scale=case.scale, **kw)
    torch.cuda.synchronize()
    return npy(out), npy(lse)


def oracle_static(case, mask=True, valid=True):
    return oracle.decode_static(npy(case.q), bits(case.k_cache), bits(case.v_cache),
                                npy(case.mask) if (mask and case.mask is not None) else None,
                                npy(case.valid_len) if (valid and case.valid_len is not None) else None,
                                case.scale)


@pytest.mark.parametrize("L", [4, 5, 103, 1152])
def test_static_tiny_matches_oracle(L):
    """Batch 1, 4 heads, head_dim 64, capacity 1152 with N(0, 10^2) garbage past L."""
    print(f"static_tiny L={L}", flush=True)
    case = workloads.static_tiny(L, device=DEV)
    out, lse = run_static(case)
    ref_out, ref_lse = oracle_static(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("D", [64, 128])
def test_static_ragged_batch_several_tiles(D):
    lengths = [1, 333, 700, 64]
    case = workloads.static_case(4, 5, D, 700, lengths, device=DEV, seed=21)
    out, lse = run_static(case)
    ref_out, ref_lse = oracle_static(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("D", [64, 128])
def test_single_row_is_bit_exact(D):
    case = workloads.static_case(2, 3, D, 256, [1, 1], device=DEV, seed=22)
    out, lse = run_static(case)
    v0 = bits(case.v_cache)[:, :, 0, :]
    expect = (v0.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(out, expect)
    ref_out, ref_lse = oracle_static(case)
    assert_lse_close(lse, ref_lse)


def test_mask_holes_and_each_limit_alone():
    case = workloads.static_case(3, 4, 128, 512, [500, 77, 512], device=DEV, seed=23,
                                 mask_density=0.6)
    out, lse = run_static(case)
    ref_out, ref_lse = oracle_static(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
    # the mask alone (rows past L are masked there too in this case)
    out_m, _ = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache, mask=case.mask,
                                       scale=case.scale)
    ref_m, _ = oracle_static(case, valid=False)
    assert_attention_close(npy(out_m), ref_m)
    # the valid length alone
    out_v, _ = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache,
                                       valid_len=case.valid_len, scale=case.scale)
    ref_v, _ = oracle_static(case, mask=False)
    assert_attention_close(npy(out_v), ref_v)


@pytest.mark.parametrize("poison", ["sigma100", "inf", "nan"])
def test_garbage_in_unattended_rows_is_bit_invisible(poison):
    case = workloads.static_case(2, 4, 128, 600, [450, 37], device=DEV, seed=24,
                                 mask_density=0.8)
    out0, lse0 = run_static(case)
    dead = torch.ones((2, 600), dtype=torch.bool, device=DEV)
    for b, L in enumerate(case.lengths):
        dead[b, :L] = case.mask[b, :L] == 0
    sel = dead[:, None, :, None].expand_as(case.k_cache)
    if poison == "sigma100":
        junk = (torch.randn(case.k_cache.shape, device=DEV) * 100).to(torch.bfloat16)
    elif poison == "inf":
        junk = torch.full(case.k_cache.shape, float("inf"), device=DEV, dtype=torch.bfloat16)
        junk[..., ::2] = float("-inf")
    else:
        junk = torch.full(case.k_cache.shape, float("nan"), device=DEV, dtype=torch.bfloat16)
    case.k_cache[sel] = junk[sel]
    case.v_cache[sel] = junk[sel]
    out1, lse1 = run_static(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_fully_masked_sequence_gives_zeros_and_minus_inf():
    case = workloads.static_case(2, 2, 64, 128, [0, 9], device=DEV, seed=25)
    out, lse = run_static(case)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    ref_out, ref_lse = oracle_static(case)
    assert_attention_close(out, ref_out)


def test_one_split_and_auto_splits_agree():
    case = workloads.static_case(2, 4, 128, 2048, [2048, 1500], device=DEV, seed=26)
    out_auto, lse_auto = run_static(case)
    out_one, lse_one = run_static(case, num_splits=1)
    out_many, _ = run_static(case, num_splits=32)
    assert np.max(np.abs(out_auto - out_one)) <= 1e-5 * np.max(np.abs(out_one))
    assert np.max(np.abs(out_many - out_one)) <= 1e-5 * np.max(np.abs(out_one))
    assert np.max(np.abs(lse_auto - lse_one)) <= 1e-5 * np.max(np.abs(lse_one))


def test_valid_length_beyond_capacity_is_clamped_and_flagged():
    case = workloads.static_case(1, 2, 64, 64, [64], device=DEV, seed=27)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    vl = torch.tensor([99], dtype=torch.int32, device=DEV)
    out, _ = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache, valid_len=vl,
                                     scale=case.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_VALID_LEN
    ref, _ = oracle.decode_static(npy(case.q), bits(case.k_cache), bits(case.v_cache), None,
                                  [64], case.scale)
    assert_attention_close(npy(out), ref)


# ----------------------------------------------------------------- kv_append


def test_kv_append_bit_exact_and_mask_update():
    B, H, cap, D = 3, 4, 40, 128
    g = torch.Generator(device=DEV).manual_seed(28)
    k = torch.randn((B, H, cap, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, H, cap, D), generator=g, device=DEV).to(torch.bfloat16)
    kn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
    mask = torch.zeros((B, cap), dtype=torch.int32, device=DEV)
    pos = torch.tensor([0, 17, 39], dtype=torch.int32, device=DEV)
    ek, ev, em = oracle.kv_append(bits(k), bits(v), bits(kn), bits(vn), npy(pos), npy(mask))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.kv_append(k, v, kn, vn, pos, mask, err_flag=flag)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), ek) and np.array_equal(bits(v), ev)
    assert np.array_equal(npy(mask), em)
    assert int(flag.item()) == 0


def test_kv_append_out_of_range_position_is_flagged_and_skipped():
    B, H, cap, D = 2, 2, 16, 64
    k = torch.zeros((B, H, cap, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    kn = torch.ones((B, H, D), dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([16, 3], dtype=torch.int32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    dakv.kv_append(k, v, kn, kn, pos, None, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_WRITE_POS
    assert float(k[0].abs().sum()) == 0.0
    assert float(k[1, :, 3].float().mean()) == 1.0


def test_page_progression_append_then_attend():
    """4-token prompt in a 1152-row buffer; steps n = 1..100 attend 4, 5, ..., 103 rows.

    Each step n >= 2 appends the previous token's K/V at row n + 2 (GPU kv_append),
    then attends; the mask popcount, the untouched rows and every output are checked
    against the oracle replaying the same steps."""
    B, H, cap, D, P = 1, 4, 1152, 64, 4
    g = torch.Generator(device=DEV).manual_seed(29)
    k = (torch.randn((B, H, cap, D), generator=g, device=DEV) * 10).to(torch.bfloat16)
    v = (torch.randn((B, H, cap, D), generator=g, device=DEV) * 10).to(torch.bfloat16)
    k[:, :, :P] = torch.randn((B, H, P, D), generator=g, device=DEV).to(torch.bfloat16)
    v[:, :, :P] = torch.randn((B, H, P, D), generator=g, device=DEV).to(torch.bfloat16)
    mask = torch.zeros((B, cap), dtype=torch.int32, device=DEV)
    mask[:, :P] = 1
    ok, ov, om = bits(k), bits(v), npy(mask)
    stored = P
    for n in range(1, 101):
        if n >= 2:
            kn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
            vn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
            pos = torch.tensor([stored], dtype=torch.int32, device=DEV)
            dakv.kv_append(k, v, kn, vn, pos, mask)
            ok, ov, om = oracle.kv_append(ok, ov, bits(kn), bits(vn), [stored], om)
            stored += 1
        q = torch.randn((B, H, D), generator=g, device=DEV)
        L = n + 3
        out, lse = dakv.decode_attn_static(q, k, v, mask=mask, scale=1 / 8)
        torch.cuda.synchronize()
        assert int(mask.sum()) == L == stored
        if n in (1, 2, 3, 50, 99, 100):
            assert np.array_equal(bits(k), ok) and np.array_equal(npy(mask), om)
            ref_out, ref_lse = oracle.decode_static(npy(q), ok, ov, om, None, 1 / 8)
            assert_attention_close(npy(out), ref_out)
            assert_lse_close(npy(lse), ref_lse)


# ------------------------------------------------------- LLaMA-7B-shaped step


@pytest.mark.parametrize("B", [1, 8])
def test_llama_layer_step_full_size_sampled(B):
    """Capacity 4096, 32 heads x 128, 32 layers, L_b uniform on 1..4096: append then
    attend in every layer exactly as the benchmark does; sampled (layer, b) pairs are
    checked against the oracle, all heads."""
    print(f"llama step B={B}", flush=True)
    model = workloads.static_llama_layers(B, device=DEV, seed=2)
    outs = []
    for layer in model.layers:
        dakv.kv_append(layer.k_cache, layer.v_cache, layer.k_new, layer.v_new, model.write_pos,
                       model.mask)
        out, lse = dakv.decode_attn_static(layer.q, layer.k_cache, layer.v_cache,
                                           mask=model.mask, valid_len=model.valid_len,
                                           scale=model.scale)
        outs.append((out, lse))
    torch.cuda.synchronize()
    rng = np.random.default_rng(30)
    for li in sorted({0, 31, int(rng.integers(1, 31))}):
        layer = model.layers[li]
        for b in sorted({0, B - 1}):
            L = model.lengths[b]
            kc = bits(layer.k_cache[b:b + 1, :, :L])
            vc = bits(layer.v_cache[b:b + 1, :, :L])
            ref_out, ref_lse = oracle.decode_static(npy(layer.q[b:b + 1]), kc, vc, None, [L],
                                                    model.scale)
            assert_attention_close(npy(outs[li][0][b:b + 1]), ref_out)
            assert_lse_close(npy(outs[li][1][b:b + 1]), ref_lse)
            # the appended row is the new token
            assert np.array_equal(bits(layer.k_cache[b, :, L - 1]), bits(layer.k_new[b]))
    del model
    torch.cuda.empty_cache()


def test_graph_replay_of_append_and_attend_matches_eager():
    """A 3-layer append+attend step captured as a HIP graph: every replay (with eager
    work and synchronisation between replays) gives exactly the eager outputs."""
    model = workloads.static_llama_layers(2, n_layers=3, H=8, D=128, cap=1024, device=DEV,
                                          seed=31, lengths=[1000, 77])
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(2, 8, 1024, 128), dtype=torch.uint8,
                     device=DEV)
    outs = [torch.empty((2, 8, 128), dtype=torch.float32, device=DEV) for _ in model.layers]
    lses = [torch.empty((2, 8), dtype=torch.float32, device=DEV) for _ in model.layers]

    def step():
        for i, layer in enumerate(model.layers):
            dakv.kv_append(layer.k_cache, layer.v_cache, layer.k_new, layer.v_new,
                           model.write_pos, model.mask)
            dakv.decode_attn_static(layer.q, layer.k_cache, layer.v_cache, mask=model.mask,
                                    valid_len=model.valid_len, scale=model.scale, out=outs[i],
                                    lse=lses[i], workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [(npy(o).copy(), npy(l).copy()) for o, l in zip(outs, lses)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, l) in enumerate(zip(outs, lses)):
            assert np.array_equal(npy(o), eager[i][0]), (r, i)
            assert np.array_equal(npy(l), eager[i][1]), (r, i)
        dakv.decode_attn_static(model.layers[0].q, model.layers[0].k_cache,
                                model.layers[0].v_cache, valid_len=model.valid_len,
                                scale=model.scale, workspace=ws)
        torch.cuda.synchronize()
    ref, _ = oracle.decode_static(npy(model.layers[2].q), bits(model.layers[2].k_cache),
                                  bits(model.layers[2].v_cache), npy(model.mask) * 0 + 1,
                                  model.lengths, model.scale)
    assert_attention_close(eager[2][0], ref)
    del graph


def test_many_splits_merge_and_workspace_reuse():
    """Capacity 16384 at batch 1 gives 64-row splits (up to 256 per head): the merge of
    many partials, repeated on one workspace, stays at the oracle."""
    case = workloads.static_case(1, 4, 128, 16384, [16384], device=DEV, seed=32,
                                 garbage_std=1.0)
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(1, 4, 16384, 128),
                     dtype=torch.uint8, device=DEV)
    ref_out, ref_lse = oracle_static(case)
    for n in (0, 256, 3, 0):
        out, lse = dakv.decode_attn_static(case.q, case.k_cache, case.v_cache,
                                           valid_len=case.valid_len, scale=case.scale,
                                           workspace=ws, num_splits=n)
        torch.cuda.synchronize()
        assert_attention_close(npy(out), ref_out)
        assert_lse_close(npy(lse), ref_lse)


# ------------------------------------------------------------ fused decode step


@pytest.mark.parametrize("D,lengths,cap", [(128, [1, 700, 4096, 63], 4096), (64, [5, 103], 1152)])
def test_fused_step_equals_append_then_attend_bit_for_bit(D, lengths, cap):
    B, H = len(lengths), 4
    case = workloads.static_case(B, H, D, cap, lengths, device=DEV, seed=33)
    g = torch.Generator(device=DEV).manual_seed(34)
    kn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
    pos = torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device=DEV)
    mask0 = case.mask.clone()
    mask0[torch.arange(B), pos.long()] = 0          # the append sets this bit
    k1, v1, m1 = case.k_cache.clone(), case.v_cache.clone(), mask0.clone()
    dakv.kv_append(k1, v1, kn, vn, pos, m1)
    out1, lse1 = dakv.decode_attn_static(case.q, k1, v1, mask=m1, valid_len=case.valid_len,
                                         scale=case.scale)
    k2, v2, m2 = case.k_cache.clone(), case.v_cache.clone(), mask0.clone()
    out2, lse2 = dakv.decode_step_static(case.q, k2, v2, kn, vn, pos, mask=m2,
                                         valid_len=case.valid_len, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(m1, m2)
    ek, ev, em = oracle.kv_append(bits(case.k_cache), bits(case.v_cache), bits(kn), bits(vn),
                                  npy(pos), npy(mask0))
    ref_out, ref_lse = oracle.decode_static(npy(case.q), ek, ev, em, lengths, case.scale)
    assert_attention_close(npy(out2), ref_out)
    assert_lse_close(npy(lse2), ref_lse)


def test_fused_step_position_outside_attended_rows_and_out_of_range():
    """A write position past the valid length is stored but not attended; one outside
    the buffer is flagged and the sequence is attended without it."""
    B, H, D, cap = 2, 2, 128, 512
    case = workloads.static_case(B, H, D, cap, [100, 300], device=DEV, seed=35)
    kn = torch.ones((B, H, D), dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([400, 512], dtype=torch.int32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    k0 = bits(case.k_cache).copy()
    out, _ = dakv.decode_step_static(case.q, case.k_cache, case.v_cache, kn, kn, pos,
                                     mask=case.mask, valid_len=case.valid_len, scale=case.scale,
                                     err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & dakv._lib.ERR_WRITE_POS
    assert float(case.k_cache[0, :, 400].float().mean()) == 1.0 and int(case.mask[0, 400]) == 1
    assert np.array_equal(bits(case.k_cache)[1], k0[1])
    ref, _ = oracle.decode_static(npy(case.q), k0, bits(case.v_cache), None, [100, 300],
                                  case.scale)
    assert_attention_close(npy(out), ref)


def test_largest_capacity_uses_all_256_splits():
    """Capacity 65536 (the static kernel's limit: 256 splits of 256 rows), full and
    ragged lengths; one more row than the limit is refused on the host."""
    print("static cap 65536", flush=True)
    case = workloads.static_case(2, 2, 64, 65536, [65536, 40000], device=DEV, seed=36,
                                 garbage_std=1.0)
    out, lse = run_static(case)
    ref_out, ref_lse = oracle_static(case)
    assert_attention_close(out, ref_out)
    assert_lse_close(lse, ref_lse)
    big = torch.zeros((1, 1, 65537, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        dakv.decode_attn_static(torch.zeros((1, 1, 64), device=DEV), big, big,
                                valid_len=torch.tensor([1], dtype=torch.int32, device=DEV))
