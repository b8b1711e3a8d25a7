// Decode attention, split-K over the row (sequence) axis, for the static buffer
// and the paged cache, and the log-sum-exp merge of the splits.
//
// Static layout: one workgroup (4 waves) per (sequence, head, split of `chunk`
// rows).  Paged layout: one workgroup per (sequence, split) over all KV heads
// when their count divides 16, else one per (sequence, KV head, split).  A row
// of D = 128 bf16 is 256 bytes = 16 lanes x 16 bytes, so one 128-bit load per lane
// covers 4 rows per wave (8 rows at D = 64).  Each 16-lane group keeps its own
// running max m, sum l and output o (8 dims per lane) over the rows it sees
// (online softmax in base 2: log2(e) is folded into the query), the dot product is
// reduced across the group with DPP row operations, and rows outside the attended
// set are never loaded.  For grouped-query attention each loaded K/V row serves
// all G query heads of its KV head.
//
// End of a split: in the static kernel every lane group's state goes to LDS and
// each output element combines all 16 of them after one barrier; in the paged
// kernels the groups of a wave merge through cross-lane shuffles first, the 4
// waves through LDS.  A sequence that fits one split writes out = o / l directly.
// Otherwise each split stores its normalised partial o / l and log2-sum-exp in the
// workspace and merge_kernel combines them (weights 2^(lse_j - max)).  (Merging in
// the last split to finish would need device-scope fences between workgroups; on
// this chip those write back and invalidate the L2 of the XCD, which costs far
// more than the second launch.)
#include "split_common.hpp"

namespace dakv {

// ---------------------------------------------------------------- static layout

// Split pass of decode_attn_static and, with kAppend, of decode_step_static.
// A split is kSteps steps of U rows per lane group (chunk rows).  Workgroups are
// numbered split-major (all units' first splits, then all second splits, ...).
//
// Appending: in the split that owns position p = write_pos[b], the lanes that
// later load that row's pieces load the new K/V row at the start and use it in
// place of what their load of row p returns (the old contents); they store it to
// the cache after the row loop, so the owning split (the last of its head,
// dispatched late) issues its row loads without waiting for the new row.  p is
// attended whatever its mask entry says (the append sets it), and the mask bit is
// written once per sequence.
template <int D, int U, int kSteps, bool kAppend>
__global__ void __launch_bounds__(kThreads)
static_decode_kernel(const float* __restrict__ q, uint16_t* __restrict__ k_cache,
                     uint16_t* __restrict__ v_cache, int32_t* __restrict__ mask,
                     const int32_t* __restrict__ valid_len, const uint16_t* __restrict__ k_new,
                     const uint16_t* __restrict__ v_new, const int32_t* __restrict__ write_pos,
                     int H, int cap, float scale_log2, int chunk, int units, Workspace ws,
                     float* __restrict__ out, float* __restrict__ lse, int32_t* err_flag) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int kStep = kWaves * RPW * U;             // rows per step
  constexpr int kBallots = (kSteps * kStep + 63) / 64;
  const int split = blockIdx.x / units;
  const int bh = blockIdx.x - split * units;
  const int max_splits = gridDim.x / units;
  const int b = bh / H;
  const int h = bh - b * H;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int slot = lane / LPR;
  const int r0 = split * chunk;
  const int32_t* mrow = mask ? mask + (size_t)b * cap : nullptr;
  // Every load this split needs before any wait: the valid length, the append
  // position, the query, and the mask entries of the split's rows (clamped
  // into the row, never branched).
  const int Lraw = valid_len ? valid_len[b] : cap;
  int p = kAppend ? write_pos[b] : -1;
  const float4* qp = reinterpret_cast<const float4*>(q + (size_t)bh * D + sub * 8);
  const float4 qa = qp[0], qc = qp[1];
  int32_t mv[kBallots];
  if (mrow) {
#pragma unroll
    for (int k = 0; k < kBallots; ++k) mv[k] = mrow[min(r0 + 64 * k + lane, cap - 1)];
  }
  const bool report = split == 0 && h == 0 && threadIdx.x == 0;
  bool owner = false;  // this lane loads a piece of row p in the loop below
  uint4 kn{}, vn{};
  if constexpr (kAppend) {
    if (p < 0 || p >= cap) {
      if (report) raise_flag(err_flag, 2);
      p = -1;
    } else if (p / chunk == split) {
      const int o = p - r0;  // the lanes of (wave, slot) below load row p in the loop
      owner = wave == (o / RPW) % kWaves && slot == o % RPW;
      if (owner) {
        kn = load16(k_new + (size_t)bh * D + sub * 8);
        vn = load16(v_new + (size_t)bh * D + sub * 8);
      }
      if (mrow && h == 0 && threadIdx.x == 0) mask[(size_t)b * cap + p] = 1;
    } else {
      p = -1;  // another split holds the new row
    }
  }
  auto store_new = [&]() {
    const size_t at = ((size_t)bh * cap + p) * D + (size_t)sub * 8;
    store16(k_cache + at, kn);
    store16(v_cache + at, vn);
  };
  int L = Lraw;
  if (L < 0 || L > cap) {
    if (report) raise_flag(err_flag, 16);
    L = L < 0 ? 0 : cap;
  }
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  if (split >= n) {
    if (kAppend && owner) store_new();  // a row past the attended ones is still stored
    return;
  }
  const int r1 = min(r0 + chunk, L);
  float qr[1][8];
  qr[0][0] = qa.x * scale_log2; qr[0][1] = qa.y * scale_log2;
  qr[0][2] = qa.z * scale_log2; qr[0][3] = qa.w * scale_log2;
  qr[0][4] = qc.x * scale_log2; qr[0][5] = qc.y * scale_log2;
  qr[0][6] = qc.z * scale_log2; qr[0][7] = qc.w * scale_log2;
  // bit (t - r0) of the ballots: row t of the split is attended
  uint64_t bits[kBallots];
#pragma unroll
  for (int k = 0; k < kBallots; ++k)
    bits[k] = __ballot(r0 + 64 * k + lane < r1 && (!mrow || mv[k] != 0));
  const BufferRows rows(k_cache + (size_t)bh * cap * D, v_cache + (size_t)bh * cap * D,
                        (uint32_t)cap * D * 2);
  const uint32_t lane_off = (uint32_t)sub * 16;
  auto row_at = [&](int t, bool& ok) -> uint32_t {
    const int o = t - r0;
    ok = ok && (((bits[o >> 6] >> (o & 63)) & 1ull) || t == p);
    return ok ? (uint32_t)t * (D * 2) + lane_off : BufferRows::kNoRow;
  };
  auto patch = [&](int t, uint4& kr, uint4& vr) {
    if (kAppend && t == p) {  // only the owning lanes meet row p
      kr = kn;
      vr = vn;
    }
  };
  HeadState<1> st;
  init_state(st);
  attend_rows_fixed<D, 1, U, kSteps>(rows, qr, r0, r1, wave, slot, row_at, patch, st);
  if (kAppend && owner) store_new();
  finish_split_flat<D>(st, lane, wave, ws, (size_t)bh, split, n, max_splits, out, lse);
}

// ------------------------------------------------------------------ paged layout
template <int G>
constexpr int paged_super_rows() {
  return kWaves * 4 * PagedShape<G>::U * PagedShape<G>::kSteps;  // D = 128: 4 rows per wave
}

template <int G>
__global__ void __launch_bounds__(kThreads)
paged_decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ key_cache,
                    const uint16_t* __restrict__ value_cache,
                    const int32_t* __restrict__ block_tables, int table_cols,
                    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
                    int Hq, int Hkv, int num_blocks, int block_size, int bs_log2, int max_len,
                    float scale_log2, int chunk, int max_splits, Workspace ws,
                    float* __restrict__ out, float* __restrict__ lse, int32_t* err_flag) {
  constexpr int D = 128;
  constexpr int LPR = D / 8;
  constexpr int U = PagedShape<G>::U;
  constexpr int kSteps = PagedShape<G>::kSteps;
  constexpr int kSuper = paged_super_rows<G>();
  __shared__ int tbl[kMaxTableSpan];
  const int split = blockIdx.x % max_splits;
  const int bg = blockIdx.x / max_splits;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int group = Hq / Hkv;  // == G
  // the query first (independent of everything else), then the lengths
  uint4 qraw[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    qraw[j] = load16(q + ((size_t)b * Hq + (size_t)g * group + j) * D + sub * 8);
  int toff = 0;
  const int L = paged_len(seq_lens, seq_offset, b, block_size, table_cols, max_len, &toff,
                          err_flag, split == 0 && g == 0 && threadIdx.x == 0);
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  if (split >= n) return;
  const int r0 = split * chunk;
  const int r1 = min(r0 + chunk, L);
  const int blk0 = r0 >> bs_log2;
  const int nblk = r1 > r0 ? ((r1 - 1) >> bs_log2) - blk0 + 1 : 0;
  for (int i = threadIdx.x; i < nblk; i += kThreads) {
    int phys = block_tables[(size_t)b * table_cols + toff + blk0 + i];
    if (phys < 0 || phys >= num_blocks) {
      raise_flag(err_flag, 1);
      phys = -1;
    }
    tbl[i] = phys;
  }
  float qr[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    unpack8(qraw[j], qr[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[j][i] *= scale_log2;
  }
  __syncthreads();
  const size_t row_stride = (size_t)Hkv * D;
  const size_t head_off = (size_t)g * D + (size_t)sub * 8;
  const int bs_mask = block_size - 1;
  const GlobalRows rows{key_cache, value_cache};
  auto row_at = [&](int t, bool& ok) -> size_t {
    const int phys = ok ? tbl[(t >> bs_log2) - blk0] : -1;
    ok = phys >= 0;
    return ok ? ((size_t)phys * block_size + (t & bs_mask)) * row_stride + head_off : 0;
  };
  HeadState<G> st;
  init_state(st);
  for (int base = r0; base < r1; base += kSuper)
    attend_rows_fixed<D, G, U, kSteps>(rows, qr, base, r1, wave, lane / LPR, row_at, NoPatch{},
                                       st);
  merge_groups<LPR, G>(st);
  finish_split<D, G>(st, lane, wave, ws, (size_t)b * Hq + (size_t)g * group, split, n,
                     max_splits, out, lse);
}

// ---------------------------------------------------------- paged, all heads
// Paged decode with one workgroup per (sequence, split) over every KV head, for
// Hkv dividing 16.  The 16 lane groups of a workgroup (4 waves x 4 groups of 16
// lanes) are numbered gi = 4 * wave + lane / 16; group gi serves KV head gi % Hkv
// at token slot gi / Hkv, so one load of every group covers TS = 16 / Hkv whole
// token rows of the block (all Hkv heads of a row are Hkv * 256 contiguous
// bytes), and a super-step reads whole blocks instead of one head's 256-byte
// piece of each row.  Group gi attends tokens slot, slot + TS, slot + 2 TS, ...
// of the split; the TS groups of one head are merged through LDS at the end.
template <int D, int U, typename RowAt>
__device__ __forceinline__ void issue_slots(const GlobalRows& rows, int t0, int ts, int r1,
                                            RowAt& row_at, uint4 (&kr)[U], uint4 (&vr)[U],
                                            bool (&ok)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u * ts;
    ok[u] = t < r1;
    const size_t off = row_at(t, ok[u]);
    rows.load(off, ok[u], kr[u], vr[u]);
  }
}

// As attend_rows_fixed, for a lane group that takes every ts-th token from t0.
template <int D, int G, int U, int kSteps, typename RowAt>
__device__ __forceinline__ void attend_slots_fixed(const GlobalRows& rows, const float (&q)[G][8],
                                                   int t0, int ts, int r1, RowAt row_at,
                                                   HeadState<G>& st) {
  const int step = U * ts;
  uint4 kr[2][U], vr[2][U];
  bool ok[2][U];
  issue_slots<D, U>(rows, t0, ts, r1, row_at, kr[0], vr[0], ok[0]);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s + 1 < kSteps)
      issue_slots<D, U>(rows, t0 + (s + 1) * step, ts, r1, row_at, kr[(s + 1) & 1],
                        vr[(s + 1) & 1], ok[(s + 1) & 1]);
    consume_rows<D, G, U>(q, kr[s & 1], vr[s & 1], ok[s & 1], st);
  }
}

template <int G>
__global__ void __launch_bounds__(kThreads)
paged_rows_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ key_cache,
                  const uint16_t* __restrict__ value_cache,
                  const int32_t* __restrict__ block_tables, int table_cols,
                  const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
                  int Hkv, int num_blocks, int block_size, int bs_log2, int max_len,
                  float scale_log2, int chunk, int max_splits, Workspace ws,
                  float* __restrict__ out, float* __restrict__ lse, int32_t* err_flag) {
  constexpr int D = 128;
  constexpr int LPR = D / 8;
  constexpr int U = PagedShape<G>::U;
  constexpr int kSteps = PagedShape<G>::kSteps;
  __shared__ int tbl[kMaxTableSpan];
  const int split = blockIdx.x % max_splits;
  const int b = blockIdx.x / max_splits;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int gi = wave * 4 + lane / LPR;
  const int ts = kRowGroups / Hkv;
  const int h = gi % Hkv;
  const int slot = gi / Hkv;
  const int Hq = Hkv * G;
  uint4 qraw[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    qraw[j] = load16(q + ((size_t)b * Hq + (size_t)h * G + j) * D + sub * 8);
  int toff = 0;
  const int L = paged_len(seq_lens, seq_offset, b, block_size, table_cols, max_len, &toff,
                          err_flag, split == 0 && threadIdx.x == 0);
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  if (split >= n) return;
  const int r0 = split * chunk;
  const int r1 = min(r0 + chunk, L);
  const int blk0 = r0 >> bs_log2;
  const int nblk = r1 > r0 ? ((r1 - 1) >> bs_log2) - blk0 + 1 : 0;
  for (int i = threadIdx.x; i < nblk; i += kThreads) {
    int phys = block_tables[(size_t)b * table_cols + toff + blk0 + i];
    if (phys < 0 || phys >= num_blocks) {
      raise_flag(err_flag, 1);
      phys = -1;
    }
    tbl[i] = phys;
  }
  float qr[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    unpack8(qraw[j], qr[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[j][i] *= scale_log2;
  }
  __syncthreads();
  const size_t row_stride = (size_t)Hkv * D;
  const size_t head_off = (size_t)h * D + (size_t)sub * 8;
  const int bs_mask = block_size - 1;
  const GlobalRows rows{key_cache, value_cache};
  auto row_at = [&](int t, bool& ok) -> size_t {
    const int phys = ok ? tbl[(t >> bs_log2) - blk0] : -1;
    ok = phys >= 0;
    return ok ? ((size_t)phys * block_size + (t & bs_mask)) * row_stride + head_off : 0;
  };
  HeadState<G> st;
  init_state(st);
  const int super = ts * U * kSteps;
  for (int base = r0; base < r1; base += super)
    attend_slots_fixed<D, G, U, kSteps>(rows, qr, base + slot, ts, r1, row_at, st);
  finish_split_rows<G>(st, gi, sub, Hkv, ts, ws, (size_t)b * Hq, split, n, max_splits, out, lse);
}

// ------------------------------------------------------------------- merge
// One workgroup per (sequence, query head); heads that fit one split return at
// once.  Length modes: 0 = static (valid_len or cap), 1 = paged.
template <int D>
__global__ void __launch_bounds__(kThreads)
merge_kernel(Workspace ws, int heads, int chunk, int max_splits, int mode,
             const int32_t* __restrict__ valid_len, int cap, const int32_t* __restrict__ seq_lens,
             const int32_t* __restrict__ seq_offset, int block_size, int table_cols, int max_len,
             float* __restrict__ out, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / heads;
  int L, toff;
  bool bad;
  if (mode == 0) {
    L = valid_len ? valid_len[b] : cap;
    L = L < 0 ? 0 : (L > cap ? cap : L);
  } else {
    L = paged_len_of(seq_lens[b], seq_lens[b + 1], seq_offset ? seq_offset[b] : 0, block_size,
                     table_cols, max_len, &toff, &bad);
  }
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  if (n == 1) return;  // the split kernel wrote this head's output
  merge_head<D>(ws.lse + (size_t)bh * max_splits, ws.o + (size_t)bh * max_splits * D, n,
                out + (size_t)bh * D, lse ? lse + bh : nullptr);
}

hipError_t launch_static_merge(const Workspace& w, int B, int H, int D, int chunk,
                               int max_splits, const int32_t* valid_len, int cap, float* out,
                               float* lse, hipStream_t stream) {
  if (D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(B * H), dim3(kThreads), 0, stream, w, H, chunk,
                       max_splits, 0, valid_len, cap, nullptr, nullptr, 1, 0, 0, out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(B * H), dim3(kThreads), 0, stream, w, H, chunk,
                       max_splits, 0, valid_len, cap, nullptr, nullptr, 1, 0, 0, out, lse);
  return hipGetLastError();
}

hipError_t launch_paged_merge(const Workspace& w, int B, int Hq, int chunk, int max_splits,
                              const int32_t* seq_lens, const int32_t* seq_offset,
                              int block_size, int table_cols, int max_seq_len, float* out,
                              float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel<128>, dim3(B * Hq), dim3(kThreads), 0, stream, w, Hq, chunk,
                     max_splits, 1, nullptr, 0, seq_lens, seq_offset, block_size, table_cols,
                     max_seq_len, out, lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------- planning
static int round_up(int x, int m) { return (x + m - 1) / m * m; }

SplitPlan plan_static(int B, int H, int cap, int D, int forced_splits) {
  (void)D;
  SplitPlan p;
  // at least ceil(cap / 256) rows so that the splits fit the merge's 256 slots
  int want = (cap + kMaxSplits - 1) / kMaxSplits;
  if (forced_splits > 0) {
    const int per = (cap + forced_splits - 1) / forced_splits;
    if (per > want) want = per;
  }
  // split sizes are 64, 128 or 256 rows.  Short splits (one 64-row step at
  // D = 128) let the CU hide each one's memory latency behind the others; once
  // the call has some 4096 or more 128-row splits, 128 rows measure better
  // (fewer partials to merge, fewer workgroups to launch).
  if (forced_splits <= 0 && (long long)B * H * ((cap + 127) / 128) >= 4096 && want < 128)
    want = 128;
  int c = kMinChunk;
  while (c < want && c < kStaticChunkMax) c *= 2;
  p.chunk = c;
  p.max_splits = cap > 0 ? (cap + c - 1) / c : 1;
  return p;
}

bool static_supported(int cap) { return cap > 0 && cap <= kStaticChunkMax * kMaxSplits; }

size_t static_workspace_bytes(int B, int H, int cap, int D) {
  const int splits = cap > 0 ? (cap + kMinChunk - 1) / kMinChunk : 1;
  return ws_floats((size_t)B * H, splits, D) * sizeof(float);
}

size_t static_plan_workspace_bytes(int B, int H, int D, const SplitPlan& plan) {
  return plan.max_splits > 1 ? ws_floats((size_t)B * H, plan.max_splits, D) * sizeof(float) : 0;
}


template <int D, int kSteps, bool kAppend>
static void launch_static_k(const float* q, void* k_cache, void* v_cache, int32_t* mask,
                            const int32_t* valid_len, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int B, int H, int cap, float scale,
                            float* out, float* lse, const Workspace& w, const SplitPlan& plan,
                            int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL((static_decode_kernel<D, 4, kSteps, kAppend>),
                     dim3((unsigned)(B * H * plan.max_splits)), dim3(kThreads), 0, stream, q,
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), mask,
                     valid_len, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), write_pos, H, cap, scale * kLog2e,
                     plan.chunk, B * H, w, out, lse, err_flag);
}

template <int D, bool kAppend>
static void launch_static_d(const float* q, void* k_cache, void* v_cache, int32_t* mask,
                            const int32_t* valid_len, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int B, int H, int cap, float scale,
                            float* out, float* lse, void* ws, const SplitPlan& plan,
                            int32_t* err_flag, hipStream_t stream) {
  const Workspace w = carve(ws, (size_t)B * H, plan.max_splits, D);
  constexpr int kStep = kWaves * (64 / (D / 8)) * 4;  // rows per step (U = 4)
  const int steps = (plan.chunk + kStep - 1) / kStep;
#define DAKV_STATIC(S)                                                                      \
  launch_static_k<D, S, kAppend>(q, k_cache, v_cache, mask, valid_len, k_new, v_new,         \
                                 write_pos, B, H, cap, scale, out, lse, w, plan, err_flag,   \
                                 stream)
  if (steps <= 1) DAKV_STATIC(1);
  else if (steps <= 2) DAKV_STATIC(2);
  else DAKV_STATIC(4);
#undef DAKV_STATIC
  if (plan.max_splits > 1)
    hipLaunchKernelGGL(merge_kernel<D>, dim3(B * H), dim3(kThreads), 0, stream, w, H, plan.chunk,
                       plan.max_splits, 0, valid_len, cap, nullptr, nullptr, 1, 0, 0, out, lse);
}

hipError_t launch_decode_static(const float* q, void* k_cache, void* v_cache, int32_t* mask,
                                const int32_t* valid_len, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* ws,
                                const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  const bool append = write_pos != nullptr;
  if (D == 128) {
    if (append)
      launch_static_d<128, true>(q, k_cache, v_cache, mask, valid_len, k_new, v_new, write_pos,
                                 B, H, cap, scale, out, lse, ws, plan, err_flag, stream);
    else
      launch_static_d<128, false>(q, k_cache, v_cache, mask, valid_len, k_new, v_new, write_pos,
                                  B, H, cap, scale, out, lse, ws, plan, err_flag, stream);
  } else {
    if (append)
      launch_static_d<64, true>(q, k_cache, v_cache, mask, valid_len, k_new, v_new, write_pos, B,
                                H, cap, scale, out, lse, ws, plan, err_flag, stream);
    else
      launch_static_d<64, false>(q, k_cache, v_cache, mask, valid_len, k_new, v_new, write_pos,
                                 B, H, cap, scale, out, lse, ws, plan, err_flag, stream);
  }
  return hipGetLastError();
}

static int paged_super(int G) {
  switch (G) {
    case 1: return paged_super_rows<1>();
    case 2: return paged_super_rows<2>();
    case 4: return paged_super_rows<4>();
    default: return paged_super_rows<8>();
  }
}

// The all-heads kernel serves every Hkv that divides the 16 lane groups.
static bool paged_rows(int Hkv) { return Hkv >= 1 && Hkv <= kRowGroups && kRowGroups % Hkv == 0; }

static int paged_rows_super(int G, int Hkv) {
  const int ts = kRowGroups / Hkv;
  switch (G) {
    case 1: return ts * PagedShape<1>::U * PagedShape<1>::kSteps;
    case 2: return ts * PagedShape<2>::U * PagedShape<2>::kSteps;
    case 4: return ts * PagedShape<4>::U * PagedShape<4>::kSteps;
    default: return ts * PagedShape<8>::U * PagedShape<8>::kSteps;
  }
}

SplitPlan plan_paged(int B, int Hkv, int G, int max_seq_len, int block_size,
                     int forced_splits) {
  SplitPlan p;
  const bool rows = paged_rows(Hkv);
  int unit = block_size > kMinChunk ? block_size : kMinChunk;
  const int sup = rows ? paged_rows_super(G, Hkv) : paged_super(G);
  if (sup > unit) unit = sup;
  // one split may touch at most kMaxTableSpan - 2 blocks
  const int most = ((kMaxTableSpan - 2) * block_size) / unit * unit;
  const int least = round_up((max_seq_len + kMaxSplits - 1) / kMaxSplits, unit);
  int c;
  if (forced_splits > 0) {
    c = round_up((max_seq_len + forced_splits - 1) / forced_splits, unit);
  } else if (rows) {
    // about kPagedRowsTarget workgroups if every sequence had max_seq_len rows
    const long long want = ((long long)B * max_seq_len + kPagedRowsTarget - 1) / kPagedRowsTarget;
    c = (int)(want > 1024 ? 1024 : want);
    c = round_up(c < 1 ? 1 : c, unit);
  } else {
    const long long want = ((long long)B * Hkv * max_seq_len + 4095) / 4096;
    c = (int)(want > 512 ? 512 : want);
    c = round_up(c < 1 ? 1 : c, unit);
  }
  if (c < unit) c = unit;
  if (c > most) c = most;
  if (c < least) c = least;
  p.chunk = c;
  p.max_splits = max_seq_len > 0 ? (max_seq_len + c - 1) / c : 1;
  return p;
}

bool paged_supported(int max_seq_len, int block_size) {
  // the widest super-step (128 rows) bounds the unit from below
  int unit = block_size > kMinChunk ? block_size : kMinChunk;
  if (unit < 128) unit = 128;
  const int most = ((kMaxTableSpan - 2) * block_size) / unit * unit;
  return (long long)most * kMaxSplits >= max_seq_len;
}

size_t paged_workspace_bytes(int B, int Hq, int D, int max_seq_len, int block_size) {
  const int unit = block_size > kMinChunk ? block_size : kMinChunk;
  const int least = round_up((max_seq_len + kMaxSplits - 1) / kMaxSplits, unit);
  const int c = least > unit ? least : unit;
  const int splits = max_seq_len > 0 ? (max_seq_len + c - 1) / c : 1;
  // the matrix-core kernel's pieces: up to one more per head, and a count per
  // (sequence, head group)
  return ws_floats((size_t)B * Hq, splits + 1, D) * sizeof(float) +
         (size_t)B * Hq * sizeof(int32_t);
}

hipError_t launch_decode_paged(const void* q, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse, void* ws,
                               const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  (void)D;
  const Workspace w = carve(ws, (size_t)B * Hq, plan.max_splits, 128);
  const float scale_log2 = scale * kLog2e;
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(key_cache);
  const auto* vc = static_cast<const uint16_t*>(value_cache);
  const int G = Hq / Hkv;
  if (paged_rows(Hkv)) {
    const dim3 grid((unsigned)(B * plan.max_splits));
#define DAKV_PAGED_ROWS(GG)                                                                   \
  hipLaunchKernelGGL(paged_rows_kernel<GG>, grid, dim3(kThreads), 0, stream, qb, kc, vc,     \
                     block_tables, table_cols, seq_lens, seq_offset, Hkv, num_blocks,        \
                     block_size, bs_log2, max_seq_len, scale_log2, plan.chunk,               \
                     plan.max_splits, w, out, lse, err_flag)
    switch (G) {
      case 1: DAKV_PAGED_ROWS(1); break;
      case 2: DAKV_PAGED_ROWS(2); break;
      case 4: DAKV_PAGED_ROWS(4); break;
      case 8: DAKV_PAGED_ROWS(8); break;
      default: return hipErrorInvalidValue;
    }
#undef DAKV_PAGED_ROWS
  } else {
    const dim3 grid((unsigned)(B * Hkv * plan.max_splits));
#define DAKV_PAGED(GG)                                                                        \
  hipLaunchKernelGGL(paged_decode_kernel<GG>, grid, dim3(kThreads), 0, stream, qb, kc, vc,   \
                     block_tables, table_cols, seq_lens, seq_offset, Hq, Hkv, num_blocks,    \
                     block_size, bs_log2, max_seq_len, scale_log2, plan.chunk,               \
                     plan.max_splits, w, out, lse, err_flag)
    switch (G) {
      case 1: DAKV_PAGED(1); break;
      case 2: DAKV_PAGED(2); break;
      case 4: DAKV_PAGED(4); break;
      case 8: DAKV_PAGED(8); break;
      default: return hipErrorInvalidValue;
    }
#undef DAKV_PAGED
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.max_splits <= 1) return err;
  return launch_paged_merge(w, B, Hq, plan.chunk, plan.max_splits, seq_lens, seq_offset,
                            block_size, table_cols, max_seq_len, out, lse, stream);
}

}  // namespace dakv
