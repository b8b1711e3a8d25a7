"""GPU parity of the decode steps at the exact shape and launch form the benchmark times.

The LLaMA-7B-shaped static step: batch 8, 32 heads x 128, capacity 4096, valid lengths
uniform on 1..4096 (seed 2, the benchmark's draw), 32 layers of decode_step_static
(append of the new token at row L - 1 and attention over L rows in one split pass)
captured as a HIP graph and replayed.  At this size the split pass takes 128-row splits
(two 64-row steps), the instantiation the benchmark's headline times and no smaller
case reaches.  The step follows the NPU article's generate loop (Part 2: only the new
row is written into the preallocated cache, then incremental SDPA over the stored rows)
and its Part 4 (the same command list replayed every token).

Checked: every replay bit-identical to the eager fused step; the fused step
bit-identical to the two calls kv_append + decode_attn_static on the same state;
every sequence of the first and last layers (and two more pairs) against
oracle.kv_append followed by oracle.decode_static on the pre-step state; rows other
than L - 1 untouched.  The FP8
and FP4 caches run the same check with their fused step at the same shape (4 layers).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import decode_attention_kv_amd as dakv
from conftest import assert_attention_close, assert_lse_close, bits, npy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, H, D, CAP = 8, 32, 128, 4096


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def sampled_pairs(n_layers, lengths, seed):
    """Every sequence of the first and the last layer, the longest one in the middle
    layer, and one more drawn pair."""
    rng = np.random.default_rng(seed)
    longest = int(np.argmax(lengths))
    pairs = {(0, b) for b in range(B)} | {(n_layers - 1, b) for b in range(B)}
    pairs |= {(n_layers // 2, longest), (int(rng.integers(0, n_layers)), int(rng.integers(0, B)))}
    return sorted(pairs)


def test_bf16_static_step_batch8_graph_full_size():
    print("headline bf16 step B=8 H=32 cap=4096 x32 layers", flush=True)
    assert dakv.decode_attn_static_split_rows(B, H, CAP, D) == 128
    model = workloads.static_llama_layers(B, device=DEV, seed=2)
    lengths = model.lengths
    pairs = sampled_pairs(len(model.layers), lengths, 41)
    pre = {}
    for li, b in pairs:
        layer = model.layers[li]
        pre[(li, b)] = (layer.k_cache[b].clone(), layer.v_cache[b].clone())
    mask0 = npy(model.mask).copy()
    outs = [torch.empty((B, H, D), dtype=torch.float32, device=DEV) for _ in model.layers]
    lses = [torch.empty((B, H), dtype=torch.float32, device=DEV) for _ in model.layers]
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(B, H, CAP, D), dtype=torch.uint8,
                     device=DEV)

    def step():
        for i, layer in enumerate(model.layers):
            dakv.decode_step_static(layer.q, layer.k_cache, layer.v_cache, layer.k_new,
                                    layer.v_new, model.write_pos, model.mask, model.valid_len,
                                    scale=model.scale, out=outs[i], lse=lses[i], workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [(npy(o).copy(), npy(l).copy()) for o, l in zip(outs, lses)]
    graph = capture(step)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, l) in enumerate(zip(outs, lses)):
            assert np.array_equal(npy(o), eager[i][0]), (r, i)
            assert np.array_equal(npy(l), eager[i][1]), (r, i)
        # eager work between replays, on the same workspace
        dakv.decode_attn_static(model.layers[1].q, model.layers[1].k_cache,
                                model.layers[1].v_cache, valid_len=model.valid_len,
                                scale=model.scale, workspace=ws)
        torch.cuda.synchronize()
    del graph
    # the same state through the two calls (the append rewrites the same rows)
    for i, layer in enumerate(model.layers):
        dakv.kv_append(layer.k_cache, layer.v_cache, layer.k_new, layer.v_new, model.write_pos,
                       model.mask)
        o2, l2 = dakv.decode_attn_static(layer.q, layer.k_cache, layer.v_cache,
                                         mask=model.mask, valid_len=model.valid_len,
                                         scale=model.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(npy(o2), eager[i][0]) and np.array_equal(npy(l2), eager[i][1]), i
    for (li, b) in pairs:
        layer = model.layers[li]
        L = lengths[b]
        k_pre, v_pre = pre[(li, b)]
        # rows other than the appended one are untouched
        keep = torch.ones(CAP, dtype=torch.bool, device=DEV)
        keep[L - 1] = False
        assert torch.equal(layer.k_cache[b][:, keep].view(torch.int16),
                           k_pre[:, keep].view(torch.int16))
        assert torch.equal(layer.v_cache[b][:, keep].view(torch.int16),
                           v_pre[:, keep].view(torch.int16))
        ek, ev, em = oracle.kv_append(bits(k_pre[None, :, :L]), bits(v_pre[None, :, :L]),
                                      bits(layer.k_new[b:b + 1]), bits(layer.v_new[b:b + 1]),
                                      [L - 1], mask0[b:b + 1, :L])
        assert np.array_equal(em[0], np.ones(L, np.int32))
        ref_out, ref_lse = oracle.decode_static(npy(layer.q[b:b + 1]), ek, ev, em, [L],
                                                model.scale)
        assert_attention_close(eager[li][0][b:b + 1], ref_out)
        assert_lse_close(eager[li][1][b:b + 1], ref_lse)
    del model
    torch.cuda.empty_cache()


def lowbit_layers(fmt, n_layers, lengths, seed):
    per = 2 if fmt == "fp4" else 1
    g = torch.Generator(device=DEV).manual_seed(seed)
    lo, hi = (-12, -5) if fmt == "fp8" else (-3, 1)
    layers = []
    for _ in range(n_layers):
        kc = torch.randint(0, 256, (B, H, CAP, D // per), generator=g, device=DEV,
                           dtype=torch.uint8)
        vc = torch.randint(0, 256, (B, H, CAP, D // per), generator=g, device=DEV,
                           dtype=torch.uint8)
        if fmt == "fp8":
            for c in (kc, vc):
                c[(c & 0x7F) == 0x7F] = 0x7E
        ks = torch.exp2(torch.randint(lo, hi, (B, H, CAP), generator=g, device=DEV).float())
        vs = torch.exp2(torch.randint(lo, hi, (B, H, CAP), generator=g, device=DEV).float())
        q = torch.randn((B, H, D), generator=g, device=DEV) * (0.5 if fmt == "fp8" else 0.1)
        kn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
        vn = torch.randn((B, H, D), generator=g, device=DEV).to(torch.bfloat16)
        layers.append([q, kc, vc, ks, vs, kn, vn])
    return layers


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_lowbit_static_step_batch8_graph_full_size(fmt):
    print(f"headline {fmt} step B=8 H=32 cap=4096 x4 layers", flush=True)
    n_layers = 4
    lengths = workloads.uniform_lengths(B, 1, CAP, 2)
    layers = lowbit_layers(fmt, n_layers, lengths, 43)
    mask = torch.zeros((B, CAP), dtype=torch.int32, device=DEV)
    for b, L in enumerate(lengths):
        mask[b, :L - 1] = 1
    mask0 = npy(mask).copy()
    wpos = torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device=DEV)
    vlen = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(B, H, CAP, D), dtype=torch.uint8,
                     device=DEV)
    if fmt == "fp8":
        step_fn, append_fn, attn_fn = (dakv.decode_step_static_fp8, dakv.kv_append_fp8,
                                       dakv.decode_attn_static_fp8)
        o_append, o_attn = oracle.kv_append_fp8, oracle.decode_static_fp8
    else:
        step_fn, append_fn, attn_fn = (dakv.decode_step_static_fp4, dakv.kv_append_fp4,
                                       dakv.decode_attn_static_fp4)
        o_append, o_attn = oracle.kv_append_fp4, oracle.decode_static_fp4
    pairs = sampled_pairs(n_layers, lengths, 44)
    pre = {(li, b): [npy(x[b:b + 1]).copy() for x in layers[li][1:5]] for li, b in pairs}
    outs = [torch.empty((B, H, D), dtype=torch.float32, device=DEV) for _ in layers]
    lses = [torch.empty((B, H), dtype=torch.float32, device=DEV) for _ in layers]

    def step():
        for i, (q, kc, vc, ks, vs, kn, vn) in enumerate(layers):
            step_fn(q, kc, vc, ks, vs, kn, vn, wpos, mask=mask, valid_len=vlen, out=outs[i],
                    lse=lses[i], workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [(npy(o).copy(), npy(l).copy()) for o, l in zip(outs, lses)]
    graph = capture(step)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, l) in enumerate(zip(outs, lses)):
            assert np.array_equal(npy(o), eager[i][0]), (r, i)
            assert np.array_equal(npy(l), eager[i][1]), (r, i)
    del graph
    for i, (q, kc, vc, ks, vs, kn, vn) in enumerate(layers):
        append_fn(kc, vc, ks, vs, kn, vn, wpos, mask=mask)
        o2, l2 = attn_fn(q, kc, vc, ks, vs, mask=mask, valid_len=vlen, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(npy(o2), eager[i][0]) and np.array_equal(npy(l2), eager[i][1]), i
    for (li, b) in pairs:
        q, kc, vc, ks, vs, kn, vn = layers[li]
        L = lengths[b]
        kc0, vc0, ks0, vs0 = pre[(li, b)]
        want = o_append(kc0[:, :, :L], vc0[:, :, :L], ks0[:, :, :L], vs0[:, :, :L],
                        bits(kn[b:b + 1]), bits(vn[b:b + 1]), [L - 1], mask0[b:b + 1, :L])
        # the stored codes and scales of the new row are the oracle's, the rest untouched
        got = [npy(x[b:b + 1]) for x in (kc, vc, ks, vs)]
        for g_arr, w_arr, p_arr in zip(got, want[:4], (kc0, vc0, ks0, vs0)):
            assert np.array_equal(g_arr[:, :, :L].astype(np.float64),
                                  np.asarray(w_arr, dtype=np.float64))
            assert np.array_equal(g_arr[:, :, L:], p_arr[:, :, L:])
        ref_out, ref_lse = o_attn(npy(q[b:b + 1]), *want[:4], mask=want[4], valid_len=[L])
        assert_attention_close(eager[li][0][b:b + 1], ref_out)
        assert_lse_close(eager[li][1][b:b + 1], ref_lse)
    del layers
    torch.cuda.empty_cache()
