#!/usr/bin/env python3
"""Benchmark of decode attention over a KV cache on one MI355X.

Default workload (one "step"): a LLaMA-7B-shaped decode step over the static
preallocated buffer -- 32 layers, each with its own bf16 cache [B, 32, 4096, 128];
per layer the new token's K/V is appended at row L_b - 1 (kv_append) and one
fp32 query row per head attends the L_b valid rows (decode_attn_static); L_b is
uniform on 1..4096 per sequence and the same in every layer.  Batch 8 is the
headline; batch 1 and the paged gather (cache [8192, 128, 8, 128], 32 sequences
of 1..4096 tokens) are reported in the same line.  Inputs are synthetic and
resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  value = algorithmic HBM bytes per step / seconds per step
(GB/s); the roofline object prices the dominant kernel launch against the 8 TB/s
HBM peak; cpu_baseline times the fp64 oracle on a bounded sample on the host.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step and achieved HBM GB/s (% of peak); gather GB/s"
HBM_PEAK_GBS = 8000.0
REPS = 50      # timed repetitions of every per-call leg and step distribution
WARM = 5       # untimed repetitions before them (cold caches, first-launch costs)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "static_decode_step_b8_traffic.md")
STATIC_SOURCES = ("decode_kernels.hip", "split_common.hpp", "device.hpp")
SPARSE_COUNTER_FILE = os.path.join(ROOT, "profiles", "sparse_mla_b16_kernel_trace_and_traffic.md")
SPARSE_SOURCES = ("sparse_kernels.hip", "device.hpp")


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "decode_attention_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def static_sources_sha256():
    return sources_sha256(STATIC_SOURCES)


def sparse_sources_sha256():
    return sources_sha256(SPARSE_SOURCES)


def recorded_value(path, sha_key, sha, key, kind=int):
    """A `key: value` line of a committed counter summary, or None when the file is
    missing or its `sha_key` line names other kernel sources than `sha`."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for raw in text.splitlines():
        line = raw.strip().strip("`")
        if ":" in line and line.startswith((sha_key, key)):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get(sha_key) != sha:
        return None
    try:
        return kind(fields[key])
    except (KeyError, ValueError):
        return None


def recorded_traffic():
    """HBM bytes per fused step call from the committed counter summary, or None
    when it is missing or was taken on other kernel sources than these."""
    return recorded_value(TRAFFIC_FILE, "kernel_sources_sha256", static_sources_sha256(),
                          "traffic_bytes_per_call")


def recorded_sparse_mfma_busy():
    """The sparse split kernel's MFMA-busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the
    active cycles of all SIMDs) from the committed counter summary, or None when it
    was taken on other kernel sources than these."""
    return recorded_value(SPARSE_COUNTER_FILE, "sparse_sources_sha256", sparse_sources_sha256(),
                          "sparse_split_mfma_busy", float)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate host time spent on the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the batch-1 and gather legs")
    ap.add_argument("--counter-pass", action="store_true",
                    help="no timing: a 1 GiB device copy (counter calibration), then a few "
                         "eager calls of every kernel on the benchmark inputs, for "
                         "rocprofv3 --pmc runs")
    return ap.parse_args()


def event_pair(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


class StaticStep:
    """32 layers x (kv_append + decode_attn_static) with preallocated outputs."""

    def __init__(self, B, torch, dakv, workloads, acc, seed=2, lengths=None):
        self.torch, self.dakv = torch, dakv
        self.model = workloads.static_llama_layers(B, device="cuda:0", seed=seed,
                                                   lengths=lengths)
        m = self.model
        self.outs = [torch.empty((B, m.H, m.D), dtype=torch.float32, device="cuda:0")
                     for _ in m.layers]
        nbytes = dakv.decode_attn_static_workspace_size(B, m.H, m.cap, m.D)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
        self.attn_bytes = acc.decode_static_bytes(B, m.H, m.D, m.lengths, q_elem=acc.FP32,
                                                  with_mask=True, with_lse=False)
        self.append_bytes = acc.kv_append_bytes(B, m.H, m.D, with_mask=True)
        self.step_bytes = len(m.layers) * (self.attn_bytes + self.append_bytes)

    def append(self, layer):
        m = self.model
        self.dakv.kv_append(layer.k_cache, layer.v_cache, layer.k_new, layer.v_new, m.write_pos,
                            m.mask)

    def attend(self, i, layer):
        m = self.model
        self.dakv.decode_attn_static(layer.q, layer.k_cache, layer.v_cache, mask=m.mask,
                                     valid_len=m.valid_len, scale=m.scale, out=self.outs[i],
                                     workspace=self.ws, want_lse=False)

    def step(self, i, layer):
        """kv_append + decode_attn_static of one layer as one fused pass."""
        m = self.model
        self.dakv.decode_step_static(layer.q, layer.k_cache, layer.v_cache, layer.k_new,
                                     layer.v_new, m.write_pos, m.mask, m.valid_len,
                                     scale=m.scale, out=self.outs[i], workspace=self.ws,
                                     want_lse=False)

    def run(self):
        for i, layer in enumerate(self.model.layers):
            self.step(i, layer)

    def run_unfused(self):
        for i, layer in enumerate(self.model.layers):
            self.append(layer)
            self.attend(i, layer)

    def capture(self, fn):
        """fn captured once into a HIP graph (torch.cuda.CUDAGraph) after a warm-up."""
        torch = self.torch
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

    def attend_all(self):
        for i, layer in enumerate(self.model.layers):
            self.attend(i, layer)

    def append_all(self):
        for layer in self.model.layers:
            self.append(layer)

    def step_all(self):
        for i, layer in enumerate(self.model.layers):
            self.step(i, layer)

    def per_launch_ms(self, reps=10):
        """Average duration of one fused step call (split + merge kernels), one
        decode_attn_static call and one kv_append call: a graph of the 32 layers'
        calls of one kind, timed with HIP events on the stream it replays on,
        divided by 32 (gaps between the launches included)."""
        torch = self.torch
        res = []
        for fn in (self.step_all, self.attend_all, self.append_all):
            g = self.capture(fn)
            g.replay()
            torch.cuda.synchronize()
            s, e = event_pair(torch)
            s.record()
            for _ in range(reps):
                g.replay()
            e.record()
            torch.cuda.synchronize()
            res.append(s.elapsed_time(e) / reps / len(self.model.layers))
        return res[0], res[1], res[2]


def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = event_pair(torch)
    t0 = time.perf_counter()
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


def step_stats(torch, fn, reps=REPS, warm=WARM):
    """Duration statistics of individual runs of fn (one HIP event pair each, back to
    back on the current stream)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        a, b = event_pair(torch)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return stats_ms([x.elapsed_time(y) for x, y in pairs])


def tiny_leg(torch, dakv, workloads, acc):
    """The tiny static config (batch 1, 4 heads, head_dim 64, capacity 1152, N(0, 10^2)
    garbage past L): one decode_attn_static call per L, cold last-level cache.  Its
    bytes are far below what launch latency hides, so it is reported, not graded."""
    res = {}
    for L in (4, 5, 103, 1152):
        case = workloads.static_tiny(L, device="cuda:0")
        out = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda:0")
        ws = torch.zeros(dakv.decode_attn_static_workspace_size(1, 4, 1152, 64),
                         dtype=torch.uint8, device="cuda:0")
        call = lambda: dakv.decode_attn_static(case.q, case.k_cache, case.v_cache,
                                               mask=case.mask, valid_len=case.valid_len,
                                               scale=case.scale, out=out, workspace=ws,
                                               want_lse=False)
        st = time_cold(torch, call)
        nbytes = acc.decode_static_bytes(1, 4, 64, [L], q_elem=acc.FP32, with_mask=True,
                                         with_lse=False)
        res[f"L{L}"] = {**us(st), "algorithmic_bytes": nbytes}
        del case, out, ws
    return {"workload": "static-buffer decode, tiny: batch 1, 4 heads, head_dim 64, "
                        "capacity 1152 (1024 + 128), one decode_attn_static call", **res}


def batch1_legs(torch, dakv, workloads, acc, seeds=range(11, 19)):
    """The LLaMA-7B-shaped step at batch 1: the pinned full-context case (L = 4096, the
    pages' 64 MiB-per-layer / 2 GiB-per-token LLaMA-7B example) and eight drawn lengths
    (seeds 11..18), each a 32-layer fused step replayed as a HIP graph; the draws are
    reported bytes-weighted (total bytes / total time)."""
    def one(lengths=None, seed=12):
        s1 = StaticStep(1, torch, dakv, workloads, acc, seed=seed, lengths=lengths)
        g1 = s1.capture(s1.run)
        st = step_stats(torch, g1.replay)
        f1, a1, ap1 = s1.per_launch_ms()
        r = {**us(st, "us_per_step"), "valid_length": s1.model.lengths[0],
             "algorithmic_bytes_per_step": s1.step_bytes,
             "GBps": round(s1.step_bytes / (st["median"] * 1e-3) / 1e9, 1),
             "step_us_per_call": round(f1 * 1e3, 2), "attn_us_per_call": round(a1 * 1e3, 2),
             "kv_append_us_per_call": round(ap1 * 1e3, 2)}
        del g1, s1
        torch.cuda.empty_cache()
        return r
    pinned = one(lengths=[4096])
    draws, tb, tt = [], 0, 0.0
    for seed in seeds:
        r = one(seed=seed)
        draws.append({"seed": seed, "valid_length": r["valid_length"],
                      "us_per_step": r["us_per_step"], "GBps": r["GBps"]})
        tb += r["algorithmic_bytes_per_step"]
        tt += r["us_per_step"] * 1e-6
    pinned["frac_of_peak"] = round(pinned["GBps"] / HBM_PEAK_GBS, 4)
    return {"pinned_L4096": pinned,
            "seeds_11_18": {"draws": draws, "bytes_weighted_GBps": round(tb / tt / 1e9, 1),
                            "bytes_weighted_frac_of_peak": round(tb / tt / 1e9 / HBM_PEAK_GBS, 4),
                            "mean_us_per_step": round(tt / len(draws) * 1e6, 1)}}


def gather_leg(torch, dakv, workloads, acc, counter_pass=False):
    case = workloads.gather_nd(device="cuda:0", seed=3)
    idx = case.index
    t = torch.from_numpy(idx.block_tables).to("cuda:0")
    s = torch.from_numpy(idx.seq_lens).to("cuda:0")
    o = torch.from_numpy(idx.seq_offset).to("cuda:0")
    T = int(idx.seq_lens[-1])
    ko = torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    vo = torch.empty_like(ko)
    dakv.validate_paged(idx.block_tables, idx.seq_lens, idx.seq_offset, 8192, 128)
    call = lambda: dakv.gather_pa_kv_cache(case.key_cache, case.value_cache, t, s, o,
                                           total_tokens=T, key_out=ko, value_out=vo,
                                           validate=False)
    if counter_pass:
        call()
        torch.cuda.synchronize()
        return acc.gather_bytes(idx.lengths, 8, 128, 8, 128, 128, with_offset=True)
    # the 247 MB read and 247 MB written fit the 256 MB last-level cache together
    # only in part; flush it between calls so that every call reads from HBM
    st = time_cold(torch, call)
    warm = time_call(torch, call)
    ms = st["median"]
    nbytes = acc.gather_bytes(idx.lengths, 8, 128, 8, 128, 128, with_offset=True)
    del case, ko, vo
    return {"workload": "gather_pa_kv_cache ND: cache [8192,128,8,128] bf16, 32 sequences "
                        "of U{1..4096} tokens, block_tables [32,64], random offsets",
            "total_tokens": T, **us(st),
            "us_per_call_back_to_back": round(warm["median"] * 1e3, 2),
            "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def fp8_leg(torch, dakv, acc, B=8, steps=10, counter_pass=False):
    """The batch-B LLaMA-7B-shaped step over an FP8 cache: 32 layers x
    decode_step_static_fp8 (append + attend in one pass), same lengths as the bf16
    step, captured as a HIP graph; the two-call form (kv_append_fp8 +
    decode_attn_static_fp8) is timed beside it.  Codes are random finite E4M3 bytes,
    scales random powers of two."""
    import workloads
    lengths = workloads.uniform_lengths(B, 1, 4096, 2)
    H, D, cap, n_layers = 32, 128, 4096, 32
    g = torch.Generator(device="cuda:0")
    g.manual_seed(9)
    layers = []
    for _ in range(n_layers):
        kc = torch.randint(0, 256, (B, H, cap, D), generator=g, device="cuda:0", dtype=torch.uint8)
        vc = torch.randint(0, 256, (B, H, cap, D), generator=g, device="cuda:0", dtype=torch.uint8)
        for c in (kc, vc):
            c[(c & 0x7F) == 0x7F] = 0x7E
        ks = torch.exp2(torch.randint(-8, 2, (B, H, cap), generator=g, device="cuda:0").float())
        vs = torch.exp2(torch.randint(-8, 2, (B, H, cap), generator=g, device="cuda:0").float())
        q = torch.randn((B, H, D), generator=g, device="cuda:0") * 0.05
        kn = torch.randn((B, H, D), generator=g, device="cuda:0").to(torch.bfloat16)
        vn = torch.randn((B, H, D), generator=g, device="cuda:0").to(torch.bfloat16)
        layers.append((q, kc, vc, ks, vs, kn, vn, torch.empty((B, H, D), device="cuda:0")))
    mask = torch.zeros((B, cap), dtype=torch.int32, device="cuda:0")
    for b, L in enumerate(lengths):
        mask[b, :L - 1] = 1
    wpos = torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device="cuda:0")
    vlen = torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(B, H, cap, D), dtype=torch.uint8,
                     device="cuda:0")

    def fused():
        for q, kc, vc, ks, vs, kn, vn, out in layers:
            dakv.decode_step_static_fp8(q, kc, vc, ks, vs, kn, vn, wpos, mask=mask,
                                        valid_len=vlen, out=out, workspace=ws, want_lse=False)

    def two_calls():
        for q, kc, vc, ks, vs, kn, vn, out in layers:
            dakv.kv_append_fp8(kc, vc, ks, vs, kn, vn, wpos, mask)
            dakv.decode_attn_static_fp8(q, kc, vc, ks, vs, mask=mask, valid_len=vlen,
                                        out=out, workspace=ws, want_lse=False)

    def graph_ms(run):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        st = step_stats(torch, graph.replay)
        del graph
        return st["median"]

    if counter_pass:
        fused()
        torch.cuda.synchronize()
        del layers
        return (acc.decode_static_fp8_bytes(B, H, D, lengths) +
                acc.kv_append_fp8_bytes(B, H, D))
    ms = graph_ms(fused)
    ms_two = graph_ms(two_calls)
    step_bytes = n_layers * (acc.decode_static_fp8_bytes(B, H, D, lengths) +
                             acc.kv_append_fp8_bytes(B, H, D))
    bf16_bytes = n_layers * (acc.decode_static_bytes(B, H, D, lengths) +
                             acc.kv_append_bytes(B, H, D))
    del layers
    return {"workload": f"static decode step over an FP8 (E4M3 + row scale) cache: 32 layers x "
                        f"decode_step_static_fp8, batch {B}, 32 heads x 128, capacity 4096, "
                        f"same lengths as the bf16 step",
            "us_per_step": round(ms * 1e3, 1),
            "us_per_step_two_calls": round(ms_two * 1e3, 1),
            "algorithmic_bytes_per_step": step_bytes,
            "GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_equivalent_GBps": round(bf16_bytes / (ms * 1e-3) / 1e9, 1)}


def fp4_leg(torch, dakv, acc, B=8, steps=10, counter_pass=False):
    """The batch-B LLaMA-7B-shaped step over an FP4 cache: 32 layers x
    decode_step_static_fp4 (append and attend in one pass), same lengths as the bf16
    step, captured as a HIP graph; also timed as kv_append_fp4 + decode_attn_static_fp4.
    Codes are random bytes (two E2M1 codes each), scales random powers of two."""
    import workloads
    lengths = workloads.uniform_lengths(B, 1, 4096, 2)
    H, D, cap, n_layers = 32, 128, 4096, 32
    g = torch.Generator(device="cuda:0")
    g.manual_seed(13)
    layers = []
    for _ in range(n_layers):
        kc = torch.randint(0, 256, (B, H, cap, D // 2), generator=g, device="cuda:0",
                           dtype=torch.uint8)
        vc = torch.randint(0, 256, (B, H, cap, D // 2), generator=g, device="cuda:0",
                           dtype=torch.uint8)
        ks = torch.exp2(torch.randint(-3, 1, (B, H, cap), generator=g, device="cuda:0").float())
        vs = torch.exp2(torch.randint(-3, 1, (B, H, cap), generator=g, device="cuda:0").float())
        q = torch.randn((B, H, D), generator=g, device="cuda:0") * 0.1
        kn = torch.randn((B, H, D), generator=g, device="cuda:0").to(torch.bfloat16)
        vn = torch.randn((B, H, D), generator=g, device="cuda:0").to(torch.bfloat16)
        layers.append((q, kc, vc, ks, vs, kn, vn, torch.empty((B, H, D), device="cuda:0")))
    mask = torch.zeros((B, cap), dtype=torch.int32, device="cuda:0")
    for b, L in enumerate(lengths):
        mask[b, :L - 1] = 1
    wpos = torch.tensor([L - 1 for L in lengths], dtype=torch.int32, device="cuda:0")
    vlen = torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    ws = torch.zeros(dakv.decode_attn_static_workspace_size(B, H, cap, D), dtype=torch.uint8,
                     device="cuda:0")

    def run_fused():
        for q, kc, vc, ks, vs, kn, vn, out in layers:
            dakv.decode_step_static_fp4(q, kc, vc, ks, vs, kn, vn, wpos, mask=mask,
                                        valid_len=vlen, out=out, workspace=ws, want_lse=False)

    def run_two():
        for q, kc, vc, ks, vs, kn, vn, out in layers:
            dakv.kv_append_fp4(kc, vc, ks, vs, kn, vn, wpos, mask)
            dakv.decode_attn_static_fp4(q, kc, vc, ks, vs, mask=mask, valid_len=vlen,
                                        out=out, workspace=ws, want_lse=False)

    def timed(run):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        st = step_stats(torch, graph.replay)
        del graph
        return st["median"]

    if counter_pass:
        run_fused()
        torch.cuda.synchronize()
        del layers
        return (acc.decode_static_fp4_bytes(B, H, D, lengths) +
                acc.kv_append_fp4_bytes(B, H, D))
    ms = timed(run_fused)
    ms_two = timed(run_two)
    step_bytes = n_layers * (acc.decode_static_fp4_bytes(B, H, D, lengths) +
                             acc.kv_append_fp4_bytes(B, H, D))
    bf16_bytes = n_layers * (acc.decode_static_bytes(B, H, D, lengths) +
                             acc.kv_append_bytes(B, H, D))
    del layers
    return {"workload": f"static decode step over an FP4 (E2M1 + row scale) cache: 32 layers x "
                        f"decode_step_static_fp4, batch {B}, 32 heads x 128, capacity 4096, "
                        f"same lengths as the bf16 step",
            "us_per_step": round(ms * 1e3, 1), "us_per_step_two_calls": round(ms_two * 1e3, 1),
            "algorithmic_bytes_per_step": step_bytes,
            "GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_equivalent_GBps": round(bf16_bytes / (ms * 1e-3) / 1e9, 1)}


def copy_leg(torch, dakv, acc, counter_pass=False):
    """The page's 7B prefill -> generate hand-over: 32 layers x K and V = 64 tensors
    [1, 32, 1024] copied into [1, 32, 1152] buffers, 1024 rows each (512 MiB)."""
    g = torch.Generator(device="cuda:0")
    g.manual_seed(8)
    src = [torch.randn((1, 32, 1024, 128), generator=g, device="cuda:0").to(torch.bfloat16)
           for _ in range(64)]
    dst = [torch.zeros((1, 32, 1152, 128), dtype=torch.bfloat16, device="cuda:0")
           for _ in range(64)]
    lens = torch.tensor([1024], dtype=torch.int32, device="cuda:0")
    mask = torch.zeros((1, 1152), dtype=torch.int32, device="cuda:0")
    call = lambda: dakv.copy_kvcache(src, dst, lens, mask=mask)
    moved = acc.copy_kvcache_bytes(32, 32, 1024, 128)
    nbytes = 2 * moved + 4 + 1152 * 4
    if counter_pass:
        call()
        torch.cuda.synchronize()
        del src, dst
        return nbytes
    st = time_cold(torch, call, graph=True)
    ms = st["median"]
    del src, dst
    return {"workload": "copy_kvcache: 64 tensors [1, 32, 1024 -> 1152, 128] bf16, 1024 rows "
                        "(512 MiB read, 512 MiB written) + mask",
            **us(st), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def as_graph(torch, call):
    """The call captured once as a HIP graph (after one eager run), so that timing a
    replay measures the GPU work and not the Python marshalling of its arguments
    (copy_kvcache builds a table of 128 tensor pointers on every call)."""
    call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    return graph


def stats_ms(samples):
    """median / p10 / p90 / mean of per-rep durations (ms), and the rep count."""
    import numpy as np
    a = np.asarray(samples, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "reps": int(a.size)}


def us(st, prefix="us_per_call"):
    """A stats_ms dict as JSON fields in microseconds (the median is the headline)."""
    return {prefix: round(st["median"] * 1e3, 2), prefix + "_p10": round(st["p10"] * 1e3, 2),
            prefix + "_p90": round(st["p90"] * 1e3, 2), prefix + "_mean": round(st["mean"] * 1e3, 2),
            "reps": st["reps"]}


def time_cold(torch, call, reps=REPS, warm=WARM, graph=False):
    """Duration statistics of one call with the last-level cache flushed before each:
    a 1 GiB buffer is read (summed) in between, which leaves only clean lines of
    that buffer in the cache, so the call neither hits its own data nor pays for
    writing back someone else's (one HIP event pair per rep on the current stream).
    The flush gives the host a head start of its duration to prepare the call; a
    call whose argument marshalling takes longer (``graph=True``) is timed as a
    replay of its graph."""
    g = as_graph(torch, call) if graph else None
    run = g.replay if graph else call
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros((), dtype=torch.float32, device="cuda:0")
    pairs = []
    for r in range(warm + reps):
        torch.sum(flush, dim=0, out=sink)
        a, b = event_pair(torch)
        a.record()
        run()
        b.record()
        if r >= warm:
            pairs.append((a, b))
    torch.cuda.synchronize()
    del flush, sink, g
    return stats_ms([x.elapsed_time(y) for x, y in pairs])


def time_call(torch, call, reps=REPS, warm=WARM):
    """Duration statistics of one call from back-to-back HIP event pairs on the
    current stream (caches warm)."""
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        a, b = event_pair(torch)
        a.record()
        call()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return stats_ms([x.elapsed_time(y) for x, y in pairs])


def ceilings(torch):
    """What the HBM delivers to plain copies on this device, for context (the bar
    stays against the 8 TB/s peak): a 1 GiB device-to-device hipMemcpyAsync (bytes
    read + written per second) and a 1 GiB fp32 sum (torch's reduction kernel; bytes
    read per second), medians of 20 event-timed runs each."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    copy = time_call(torch, lambda: b.copy_(a), reps=20, warm=3)
    del b
    f = a.view(torch.float32)
    f.fill_(1.0)
    sink = torch.zeros((), dtype=torch.float32, device="cuda:0")
    read = time_call(torch, lambda: torch.sum(f, dim=0, out=sink), reps=20, warm=3)
    del a, f, sink
    torch.cuda.empty_cache()
    props = torch.cuda.get_device_properties(0)
    clocks = device_clocks()
    return {"d2d_copy_GBps": round(2 * n / (copy["median"] * 1e-3) / 1e9, 1),
            "read_sum_GBps": round(n / (read["median"] * 1e-3) / 1e9, 1),
            "device": getattr(props, "name", ""), "arch": getattr(props, "gcnArchName", ""),
            "compute_units": getattr(props, "multi_processor_count", None),
            "hbm_bytes": getattr(props, "total_memory", None), **clocks}


def device_clocks():
    """Peak engine and memory clocks (MHz) and the memory bus width of device 0, as the
    HIP runtime reports them (hipDeviceGetAttribute), for the record; None where the
    runtime library cannot be opened."""
    import ctypes
    attrs = {"sclk_peak_MHz": 5, "mclk_peak_MHz": 60, "memory_bus_bits": 59}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return {k: None for k in attrs}
    out = {}
    for key, attr in attrs.items():
        v = ctypes.c_int(0)
        ok = hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(0)) == 0
        out[key] = (v.value // 1000 if key.endswith("MHz") else v.value) if ok else None
    return out


def paged_leg(torch, dakv, workloads, acc, counter_pass=False):
    case = workloads.paged_gqa(device="cuda:0", seed=4)
    idx = case.index
    t = torch.from_numpy(idx.block_tables).to("cuda:0")
    s = torch.from_numpy(idx.seq_lens).to("cuda:0")
    B = len(idx.lengths)
    out = torch.empty((B, case.Hq, case.D), dtype=torch.float32, device="cuda:0")
    max_len = max(idx.lengths)
    ws = torch.zeros(dakv.decode_attn_paged_workspace_size(B, case.Hq, case.D, max_len, 16),
                     dtype=torch.uint8, device="cuda:0")
    call = lambda: dakv.decode_attn_paged(case.q, case.key_cache, case.value_cache, t, s, None,
                                          max_seq_len=max_len, scale=case.scale, out=out,
                                          workspace=ws, want_lse=False)
    if counter_pass:
        call()
        torch.cuda.synchronize()
        return acc.decode_paged_bytes(idx.lengths, case.Hq, case.Hkv, case.D, 16)
    st = time_cold(torch, call)
    ms = st["median"]
    nbytes = acc.decode_paged_bytes(idx.lengths, case.Hq, case.Hkv, case.D, 16)
    del case, out, ws
    return {"workload": "paged GQA decode: batch 64, 32 query / 8 KV heads, head_dim 128, "
                        "block 16, contexts log-uniform [512, 16384]",
            "total_tokens": int(sum(idx.lengths)), **us(st),
            "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def paged_lowbit_leg(torch, dakv, workloads, acc, fmt="fp8", counter_pass=False):
    """The paged GQA config over a low-bit pool (same lengths, table and pool size):
    random finite E4M3 codes (fmt "fp8") or random bytes of two E2M1 codes ("fp4"),
    row scales random powers of two."""
    case = workloads.paged_gqa(device="cuda:0", seed=4)
    idx = case.index
    nb, bs, Hkv, D = case.key_cache.shape
    del case.key_cache, case.value_cache
    fp4 = fmt == "fp4"
    g = torch.Generator(device="cuda:0")
    g.manual_seed(13 if fp4 else 12)
    codes = []
    for _ in range(2):
        c = torch.randint(0, 256, (nb, bs, Hkv, D // 2 if fp4 else D), generator=g,
                          device="cuda:0", dtype=torch.uint8)
        if not fp4:
            c[(c & 0x7F) == 0x7F] = 0x7E
        codes.append(c)
    lo, hi = (-3, 1) if fp4 else (-12, -5)
    scales = [torch.exp2(torch.randint(lo, hi, (nb, bs, Hkv), generator=g,
                                       device="cuda:0").float()) for _ in range(2)]
    t = torch.from_numpy(idx.block_tables).to("cuda:0")
    s = torch.from_numpy(idx.seq_lens).to("cuda:0")
    B = len(idx.lengths)
    out = torch.empty((B, case.Hq, D), dtype=torch.float32, device="cuda:0")
    max_len = max(idx.lengths)
    ws = torch.zeros(dakv.decode_attn_paged_workspace_size(B, case.Hq, D, max_len, bs),
                     dtype=torch.uint8, device="cuda:0")
    fn = dakv.decode_attn_paged_fp4 if fp4 else dakv.decode_attn_paged_fp8
    call = lambda: fn(case.q, codes[0], codes[1], scales[0], scales[1], t, s, None,
                      max_seq_len=max_len, scale=case.scale, out=out, workspace=ws,
                      want_lse=False)
    nbytes = (acc.decode_paged_fp4_bytes if fp4 else acc.decode_paged_fp8_bytes)(
        idx.lengths, case.Hq, Hkv, D, bs)
    if counter_pass:
        call()
        torch.cuda.synchronize()
        return nbytes
    st = time_cold(torch, call)
    ms = st["median"]
    bf16_bytes = acc.decode_paged_bytes(idx.lengths, case.Hq, Hkv, D, bs)
    del case, codes, scales, out, ws
    name = "an FP4 pool (E2M1 two per byte" if fp4 else "an FP8 pool (E4M3"
    return {"workload": f"paged GQA decode over {name} + row scale): batch 64, "
                        "32 query / 8 KV heads, head_dim 128, block 16, contexts log-uniform "
                        "[512, 16384]",
            **us(st), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_equivalent_GBps": round(bf16_bytes / (ms * 1e-3) / 1e9, 1)}


def sparse_leg(torch, dakv, workloads, acc, counter_pass=False):
    case = workloads.sparse_mla(device="cuda:0", seed=5)
    B, Hq, d_qk = case.q.shape
    topk = case.indices.shape[1]
    out = torch.empty((B, Hq, case.d_v), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(dakv.sparse_topk_decode_attn_workspace_size(B, Hq, d_qk, case.d_v, topk),
                     dtype=torch.uint8, device="cuda:0")
    call = lambda: dakv.sparse_topk_decode_attn(case.q, case.kv, case.indices, d_v=case.d_v,
                                                sm_scale=case.sm_scale, out=out, workspace=ws,
                                                want_lse=False)
    if counter_pass:
        call()
        torch.cuda.synchronize()
        return acc.sparse_bytes(B, Hq, d_qk, case.d_v, topk)
    # the 604 MB cache exceeds the 256 MB last-level cache, but the 44 MB actually
    # touched fits: flush it between calls
    st = time_cold(torch, call)
    warm = time_call(torch, call)
    ms = st["median"]
    nbytes = acc.sparse_bytes(B, Hq, d_qk, case.d_v, topk)
    flops = acc.sparse_flops(B, Hq, d_qk, case.d_v, topk)
    del case, out, ws
    return {"workload": "top-k sparse MLA decode: batch 16, 128 heads on one latent KV, "
                        "d_qk 576 / d_v 512, context 32768, top-2048",
            **us(st), "us_per_call_warm_cache": round(warm["median"] * 1e3, 2),
            "algorithmic_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 2.5e15, 4),
            "split_kernel_mfma_busy_counter": recorded_sparse_mfma_busy(),
            "mfma_busy_source": "profiles/sparse_mla_b16_kernel_trace_and_traffic.md "
                                "(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), split "
                                "kernel only; null when taken on other kernel sources)"}


def sparse_tokens_leg(torch, dakv, workloads, acc, s_q=2):
    """The sparse MLA config with s_q q-tokens per sequence (each its own top-2048
    list over the sequence's one latent cache), e.g. a draft token verified with the
    next one."""
    case = workloads.sparse_tokens_case(16, s_q, 128, 32768, 2048, device="cuda:0", seed=7)
    B, _, Hq, d_qk = case.q.shape
    topk = case.indices.shape[2]
    out = torch.empty((B, s_q, Hq, case.d_v), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(dakv.sparse_topk_decode_attn_workspace_size(B * s_q, Hq, d_qk, case.d_v,
                                                                 topk),
                     dtype=torch.uint8, device="cuda:0")
    call = lambda: dakv.sparse_topk_attn(case.q, case.kv, case.indices, d_v=case.d_v,
                                         sm_scale=case.sm_scale, out=out, workspace=ws,
                                         want_lse=False)
    st = time_cold(torch, call)
    ms = st["median"]
    nbytes = acc.sparse_bytes(B * s_q, Hq, d_qk, case.d_v, topk)
    flops = acc.sparse_flops(B * s_q, Hq, d_qk, case.d_v, topk)
    del case, out, ws
    return {"workload": f"top-k sparse MLA, {s_q} q-tokens per sequence: batch 16, 128 heads, "
                        f"d_qk 576 / d_v 512, context 32768, top-2048 per token",
            **us(st), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 2.5e15, 4)}


def sparse_lowbit_leg(torch, dakv, workloads, acc, fmt="fp8", counter_pass=False):
    """The sparse MLA config over a low-bit latent cache: E4M3 (fmt "fp8") or E2M1 two
    per byte ("fp4") codes with one power-of-two scale per latent row."""
    make = workloads.sparse_fp8_case if fmt == "fp8" else workloads.sparse_fp4_case
    fn = dakv.sparse_topk_attn_fp8 if fmt == "fp8" else dakv.sparse_topk_attn_fp4
    nbytes_of = acc.sparse_fp8_bytes if fmt == "fp8" else acc.sparse_fp4_bytes
    case = make(16, 1, 128, 32768, 2048, device="cuda:0", seed=5)
    B, s_q, Hq, d_qk = case.q.shape
    topk = case.indices.shape[2]
    out = torch.empty((B, s_q, Hq, case.d_v), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(dakv.sparse_topk_decode_attn_workspace_size(B, Hq, d_qk, case.d_v, topk),
                     dtype=torch.uint8, device="cuda:0")
    call = lambda: fn(case.q, case.codes, case.scale, case.indices, d_v=case.d_v,
                      sm_scale=case.sm_scale, out=out, workspace=ws, want_lse=False)
    nbytes = nbytes_of(B, Hq, d_qk, case.d_v, topk)
    if counter_pass:
        call()
        torch.cuda.synchronize()
        return nbytes
    st = time_cold(torch, call)
    ms = st["median"]
    flops = acc.sparse_flops(B, Hq, d_qk, case.d_v, topk)
    del case, out, ws
    name = "FP8 (E4M3" if fmt == "fp8" else "FP4 (E2M1, two per byte"
    return {"workload": f"top-k sparse MLA decode over an {name} + row scale) latent cache: "
                        "batch 16, 128 heads, d_qk 576 / d_v 512, context 32768, top-2048",
            **us(st), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 2.5e15, 4)}


def cpu_baseline(step, budget_s):
    """The fp64 oracle over (layer, sequence) pairs of the same step until the budget is
    spent; GB/s = algorithmic bytes of the pairs done / host seconds."""
    import numpy as np
    import oracle
    from decode_attention_kv_amd import accounting as acc

    def bits(t):
        return t.detach().cpu().contiguous().view(step.torch.int16).numpy().view(np.uint16)

    m = step.model
    done_bytes, pairs, spent = 0, 0, 0.0
    for layer in m.layers:
        for b in range(m.B):
            L = m.lengths[b]
            q = layer.q[b:b + 1].cpu().numpy()
            kc = bits(layer.k_cache[b:b + 1, :, :L])
            vc = bits(layer.v_cache[b:b + 1, :, :L])
            mask = m.mask[b:b + 1, :L].cpu().numpy().copy()
            mask[0, L - 1] = 1
            t0 = time.perf_counter()
            oracle.kv_append(kc, vc, bits(layer.k_new[b:b + 1]), bits(layer.v_new[b:b + 1]),
                             [L - 1], mask)
            oracle.decode_static(q, kc, vc, mask, [L], m.scale)
            spent += time.perf_counter() - t0
            done_bytes += acc.decode_static_bytes(1, m.H, m.D, [L], q_elem=acc.FP32) + \
                acc.kv_append_bytes(1, m.H, m.D)
            pairs += 1
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s",
            "cores": threads if threads else cores, "host_cores_visible": cores,
            "kind": "oracle",
            "sample": f"{pairs} (layer, sequence) pairs of the batch-{m.B} step "
                      f"(append + attend, fp64 NumPy), {spent:.1f} s"}


def cpu_single_thread(torch, workloads, acc):
    """The oracle with one BLAS/OpenMP thread on bounded samples of the tiny static
    config (all four L), the gather (two sequences, their blocks copied out of the
    pool) and the sparse MLA config (one sequence); GB/s of algorithmic bytes."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    res = {}
    with threadpool_limits(limits=1):
        nbytes, spent = 0, 0.0
        for L in (4, 5, 103, 1152):
            case = workloads.static_tiny(L, device="cuda:0")
            args = (case.q.cpu().numpy(), bits(case.k_cache), bits(case.v_cache),
                    case.mask.cpu().numpy(), [L], case.scale)
            t0 = time.perf_counter()
            oracle.decode_static(*args)
            spent += time.perf_counter() - t0
            nbytes += acc.decode_static_bytes(1, 4, 64, [L], q_elem=acc.FP32, with_mask=True,
                                              with_lse=False)
        res["static_tiny"] = {"seconds": round(spent, 4), "GBps": round(nbytes / spent / 1e9, 4),
                              "sample": "one call at each L in {4, 5, 103, 1152}"}
        g = workloads.gather_nd(device="cuda:0", seed=3)
        idx = g.index
        pick = [0, 1]
        lens = [idx.lengths[q] for q in pick]
        cols = [-(-L // 128) for L in lens]
        ids = np.concatenate([idx.block_tables[q, idx.seq_offset[q] // 128:
                                               idx.seq_offset[q] // 128 + c]
                              for q, c in zip(pick, cols)])
        sel = torch.from_numpy(ids.astype(np.int64)).to("cuda:0")
        kc, vc = bits(g.key_cache.index_select(0, sel)), bits(g.value_cache.index_select(0, sel))
        del g
        tables = np.full((len(pick), max(cols)), 0, dtype=np.int32)
        at = 0
        for i, c in enumerate(cols):
            tables[i, :c] = np.arange(at, at + c)
            at += c
        seq_lens = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        t0 = time.perf_counter()
        oracle.gather_pa_kv_cache(kc, vc, tables, seq_lens, None)
        spent = time.perf_counter() - t0
        nbytes = acc.gather_bytes(lens, 8, 128, 8, 128, 128, with_offset=False)
        res["gather_nd"] = {"seconds": round(spent, 4), "GBps": round(nbytes / spent / 1e9, 4),
                            "sample": f"2 of 32 sequences ({sum(lens)} tokens)"}
        sp = workloads.sparse_mla(device="cuda:0", seed=5)
        q, kv, ind = bits(sp.q[:1]), bits(sp.kv[:1]), sp.indices[:1].cpu().numpy()
        d_v, sm = sp.d_v, sp.sm_scale
        del sp
        t0 = time.perf_counter()
        oracle.sparse_topk_decode(q, kv, ind, d_v, sm)
        spent = time.perf_counter() - t0
        nbytes = acc.sparse_bytes(1, 128, 576, 512, 2048)
        res["sparse_mla"] = {"seconds": round(spent, 4), "GBps": round(nbytes / spent / 1e9, 4),
                             "TFLOPs": round(acc.sparse_flops(1, 128, 576, 512, 2048) / spent
                                             / 1e12, 6),
                             "sample": "1 of 16 sequences (128 heads, top-2048)"}
    torch.cuda.empty_cache()
    return {"threads": 1, **res}


def counter_pass(torch, dakv, workloads, acc, B, calls=3):
    """Launches for hardware-counter runs: a plain 1 GiB copy first (its FETCH_SIZE
    and WRITE_SIZE give the counters' scale), then `calls` eager fused steps of the
    batch-B benchmark step and one call (the low-bit steps: one step of 32 calls) of
    each other leg.  Prints the algorithmic bytes per call of each launch kind."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    step = StaticStep(B, torch, dakv, workloads, acc)
    for _ in range(calls):
        step.run()
    torch.cuda.synchronize()
    info = {"copy_bytes_each_way": 1 << 30, "static_step_call_bytes": step.attn_bytes +
            step.append_bytes, "static_step_calls": calls * len(step.model.layers),
            "static_grid_batch": B}
    del step
    torch.cuda.empty_cache()
    for name, leg in (("gather", gather_leg), ("paged_gqa", paged_leg), ("sparse_mla", sparse_leg)):
        info[name + "_call_bytes"] = leg(torch, dakv, workloads, acc, counter_pass=True)
        torch.cuda.empty_cache()
    info["copy_kvcache_call_bytes"] = copy_leg(torch, dakv, acc, counter_pass=True)
    torch.cuda.empty_cache()
    info["static_fp8_step_call_bytes"] = fp8_leg(torch, dakv, acc, B, counter_pass=True)
    torch.cuda.empty_cache()
    info["static_fp4_step_call_bytes"] = fp4_leg(torch, dakv, acc, B, counter_pass=True)
    for fmt in ("fp8", "fp4"):
        torch.cuda.empty_cache()
        info[f"paged_gqa_{fmt}_call_bytes"] = paged_lowbit_leg(torch, dakv, workloads, acc, fmt,
                                                               counter_pass=True)
        torch.cuda.empty_cache()
        info[f"sparse_mla_{fmt}_call_bytes"] = sparse_lowbit_leg(torch, dakv, workloads, acc,
                                                                 fmt, counter_pass=True)
    print(json.dumps(info), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_kv_amd as dakv
    from decode_attention_kv_amd import accounting as acc
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dakv.lib()

    B = args.batch
    if args.counter_pass:
        counter_pass(torch, dakv, workloads, acc, B)
        return
    ceil = ceilings(torch)
    step = StaticStep(B, torch, dakv, workloads, acc)
    graph = step.capture(step.run)
    ms, wall = time_steps(torch, graph.replay, args.steps, args.warmup)
    dist = step_stats(torch, graph.replay)
    eager_ms, _ = time_steps(torch, step.run, max(3, args.steps // 4), 1)
    g_unf = step.capture(step.run_unfused)
    unfused_ms, _ = time_steps(torch, g_unf.replay, max(5, args.steps // 2), 2)
    del g_unf
    fused_ms, attn_ms, app_ms = step.per_launch_ms()
    value = step.step_bytes / (ms * 1e-3) / 1e9
    fused_bytes = step.attn_bytes + step.append_bytes
    fused_gbs = fused_bytes / (fused_ms * 1e-3) / 1e9
    m = step.model
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "us_per_step": round(ms * 1e3, 1),
        "us_per_step_eager_launches": round(eager_ms * 1e3, 1),
        "us_per_step_unfused": round(unfused_ms * 1e3, 1),
        "step_distribution": {**us(dist, "us_per_step"),
                              "note": "separately event-timed graph replays"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "kv_dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"static-buffer decode step, LLaMA-7B-shaped: 32 layers x (kv_append + "
                        f"decode_attn_static), batch {B}, 32 heads x 128, capacity 4096, "
                        f"L ~ U{{1..4096}} per sequence",
            "global_batch": B, "seq_len": m.cap, "valid_lengths": m.lengths,
            "parallelism": "none (one GPU)",
            "algorithmic_bytes_per_step": step.step_bytes,
        },
        "timing": "the 32-layer step is captured once as a HIP graph and replayed; "
                  "HIP events around the replays",
        "roofline": {
            "kernel": "decode_step_static: static_decode_kernel<128,4,append> split pass + "
                      "merge_kernel<128>, one call per layer; per-call time from a graph of "
                      "the 32 calls (HIP events), so the merge and launch gaps are included",
            "bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic() if B == 8 else None,
            "bytes_per_launch": fused_bytes, "us_per_launch": round(fused_ms * 1e3, 2),
            "decode_attn_static_us_per_call": round(attn_ms * 1e3, 2),
            "kv_append_us_per_call": round(app_ms * 1e3, 2),
        },
        "wall_s_timed": round(wall, 3),
        "ceilings": ceil,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    del graph, step
    torch.cuda.empty_cache()
    if not args.no_extras:
        line["batch1"] = batch1_legs(torch, dakv, workloads, acc)
        torch.cuda.empty_cache()
        line["static_tiny"] = tiny_leg(torch, dakv, workloads, acc)
        torch.cuda.empty_cache()
        line["gather"] = gather_leg(torch, dakv, workloads, acc)
        torch.cuda.empty_cache()
        line["paged_gqa"] = paged_leg(torch, dakv, workloads, acc)
        torch.cuda.empty_cache()
        line["paged_gqa_fp8"] = paged_lowbit_leg(torch, dakv, workloads, acc, "fp8")
        torch.cuda.empty_cache()
        line["paged_gqa_fp4"] = paged_lowbit_leg(torch, dakv, workloads, acc, "fp4")
        torch.cuda.empty_cache()
        line["sparse_mla"] = sparse_leg(torch, dakv, workloads, acc)
        line["sparse_mla_2_tokens"] = sparse_tokens_leg(torch, dakv, workloads, acc)
        torch.cuda.empty_cache()
        line["sparse_mla_fp8"] = sparse_lowbit_leg(torch, dakv, workloads, acc, "fp8")
        torch.cuda.empty_cache()
        line["sparse_mla_fp4"] = sparse_lowbit_leg(torch, dakv, workloads, acc, "fp4")
        torch.cuda.empty_cache()
        line["copy_kvcache"] = copy_leg(torch, dakv, acc)
        torch.cuda.empty_cache()
        line["static_fp8"] = fp8_leg(torch, dakv, acc)
        torch.cuda.empty_cache()
        line["static_fp4"] = fp4_leg(torch, dakv, acc)
        if not args.no_cpu_baseline:
            torch.cuda.empty_cache()
            line["cpu_baseline"]["single_thread"] = cpu_single_thread(torch, workloads, acc)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
