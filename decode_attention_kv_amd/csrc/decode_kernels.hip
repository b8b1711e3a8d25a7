// Decode attention, split-K over the row (sequence) axis, for the static buffer
// and the paged cache, plus the log-sum-exp merge of the split partials.
//
// Pass 1 -- one workgroup (4 waves) per (sequence, KV head, split).  A row of
// D = 128 bf16 is 256 bytes = 16 lanes x 16 bytes, so one 128-bit load per lane
// covers 4 rows per wave (8 rows at D = 64).  Each 16-lane group keeps its own
// running max m, sum l and output o (8 dims per lane) over the rows it sees
// (online softmax, base 2: log2(e) is folded into the query), the dot product is
// reduced across the group with DPP row operations, and rows outside the
// attended set are never loaded.  At the end the groups of a wave merge through
// cross-lane shuffles, the 4 waves through LDS, and the split writes its
// normalised partial o / l and log2-sum-exp to the workspace.  For grouped-query
// attention every loaded K/V row serves all G query heads of its KV head.
//
// Pass 2 -- one workgroup per (sequence, query head): out = sum_j w_j o_j /
// sum_j w_j with w_j = 2^(lse_j - max lse); splits whose rows were all masked
// carry lse = -inf and weight 0.  With a single split this is a copy, so a lone
// attended row comes out bit-exact.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMinChunk = 64;

// Effective row count of a static-buffer sequence: valid_len[b] clamped to
// [0, cap] (clamping is flagged), or cap without a valid_len.
__device__ __forceinline__ int static_len(const int32_t* valid_len, int b, int cap,
                                          int32_t* err_flag, bool report) {
  if (!valid_len) return cap;
  int L = valid_len[b];
  if (L < 0 || L > cap) {
    if (report) raise_flag(err_flag, 16);
    L = L < 0 ? 0 : cap;
  }
  return L;
}

// Effective row count of a paged sequence: its cumulative-length difference,
// cut at max_len and at the table's last column; inconsistencies are flagged.
__device__ __forceinline__ int paged_len(const int32_t* seq_lens, const int32_t* seq_offset,
                                         int b, int block_size, int table_cols, int max_len,
                                         int* toff, int32_t* err_flag, bool report) {
  int L = seq_lens[b + 1] - seq_lens[b];
  const int off = seq_offset ? seq_offset[b] : 0;
  bool bad = false;
  if (L < 0) { L = 0; bad = true; }
  if (off < 0 || off % block_size != 0) { L = 0; bad = true; *toff = 0; }
  else *toff = off / block_size;
  const int room = (table_cols - *toff) * block_size;
  if (L > room) { L = room > 0 ? room : 0; bad = true; }
  if (L > max_len) { L = max_len; bad = true; }
  if (bad && report) raise_flag(err_flag, 8);
  return L;
}

// Online-softmax state of one query head for one 16-lane (D/8-lane) row group.
template <int G>
struct HeadState {
  float m[G], l[G], o[G][8];
};

// Merge the row groups of one wave (they differ in the lane bits above the
// group), so that every group ends with the wave's state.
template <int LPR, int G>
__device__ __forceinline__ void merge_groups(HeadState<G>& st) {
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(st.m[j], off);
      const float lo = __shfl_xor(st.l[j], off);
      const float M = fmaxf(st.m[j], mo);
      const float Ms = M == kNegInf ? 0.f : M;
      const float ws = exp2_fast(st.m[j] - Ms);
      const float wo = exp2_fast(mo - Ms);
      st.l[j] = st.l[j] * ws + lo * wo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float oo = __shfl_xor(st.o[j][i], off);
        st.o[j][i] = st.o[j][i] * ws + oo * wo;
      }
      st.m[j] = M;
    }
  }
}

// Cross-wave merge through LDS and the write of this split's partials.
// ws_o:   [unit heads][max_splits][D]  (normalised o / l)
// ws_lse: [unit heads][max_splits]     (log2 of sum 2^s, -inf if empty)
template <int D, int G>
__device__ __forceinline__ void write_partials(const HeadState<G>& st, int lane, int wave,
                                               float* __restrict__ ws_o,
                                               float* __restrict__ ws_lse, size_t head0,
                                               int split, int max_splits) {
  constexpr int LPR = D / 8;
  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_o[wave][j][lane * 8 + i] = st.o[j][i];
      if (lane == 0) {
        sm_m[wave][j] = st.m[j];
        sm_l[wave][j] = st.l[j];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int d = idx - j * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    const size_t unit = (head0 + j) * max_splits + split;
    if (M == kNegInf) {
      ws_o[unit * D + d] = 0.f;
      if (d == 0) ws_lse[unit] = kNegInf;
      continue;
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = exp2_fast(sm_m[w][j] - M);
      num += wt * sm_o[w][j][d];
      den += wt * sm_l[w][j];
    }
    ws_o[unit * D + d] = num / den;
    if (d == 0) ws_lse[unit] = M + __log2f(den);
  }
}

// The row loop shared by the static and paged kernels.  RowAt(t, ok) returns
// the element offset of row t's piece for this lane and clears ok when the row
// must not be read.  q is pre-scaled by scale * log2(e).
template <int D, int G, int U, typename RowAt>
__device__ __forceinline__ void attend_rows(const uint16_t* __restrict__ kc,
                                            const uint16_t* __restrict__ vc, const float (&q)[G][8],
                                            int r0, int r1, int wave, int slot, RowAt row_at,
                                            HeadState<G>& st) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int kStep = kWaves * RPW * U;
  for (int base = r0; base < r1; base += kStep) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + (u * kWaves + wave) * RPW + slot;
      ok[u] = t < r1;
      const size_t off = row_at(t, ok[u]);
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        kr[u] = load16(kc + off);
        vr[u] = load16(vc + off);
      }
    }
    float s[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(q[j][i], kf[i], acc);
        acc = group_sum<LPR>(acc);
        s[j][u] = ok[u] ? acc : kNegInf;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mnew = st.m[j];
#pragma unroll
      for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, s[j][u]);
      const float ms = mnew == kNegInf ? 0.f : mnew;
      const float alpha = exp2_fast(st.m[j] - ms);
      float psum = 0.f;
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = exp2_fast(s[j][u] - ms);
        psum += p[u];
      }
      st.l[j] = st.l[j] * alpha + psum;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.o[j][i] *= alpha;
      st.m[j] = mnew;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[8];
        unpack8(vr[u], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) st.o[j][i] = fmaf(p[u], vf[i], st.o[j][i]);
      }
    }
  }
}

template <int G>
__device__ __forceinline__ void init_state(HeadState<G>& st) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.o[j][i] = 0.f;
  }
}

// ---------------------------------------------------------------- static pass 1
template <int D>
__global__ void __launch_bounds__(kThreads)
static_split_kernel(const float* __restrict__ q, const uint16_t* __restrict__ k_cache,
                    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ mask,
                    const int32_t* __restrict__ valid_len, int H, int cap, float scale_log2,
                    int chunk, int max_splits, float* __restrict__ ws_o,
                    float* __restrict__ ws_lse, int32_t* err_flag) {
  constexpr int LPR = D / 8;
  constexpr int U = 4;
  const int split = blockIdx.x % max_splits;
  const int bh = blockIdx.x / max_splits;
  const int b = bh / H;
  const int L = static_len(valid_len, b, cap, err_flag, split == 0 && bh % H == 0 && threadIdx.x == 0);
  const int r0 = split * chunk;
  if (r0 >= L) return;
  const int r1 = min(r0 + chunk, L);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane / LPR;
  const int sub = lane % LPR;

  float qr[1][8];
  {
    const float* qp = q + (size_t)bh * D + sub * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[0][i] = qp[i] * scale_log2;
  }
  const size_t head_base = (size_t)bh * cap * D + (size_t)sub * 8;
  const int32_t* mrow = mask ? mask + (size_t)b * cap : nullptr;
  auto row_at = [&](int t, bool& ok) -> size_t {
    if (ok && mrow) ok = mrow[t] != 0;
    return head_base + (size_t)t * D;
  };
  HeadState<1> st;
  init_state(st);
  attend_rows<D, 1, U>(k_cache, v_cache, qr, r0, r1, wave, lane / LPR, row_at, st);
  (void)slot;
  merge_groups<LPR, 1>(st);
  write_partials<D, 1>(st, lane, wave, ws_o, ws_lse, (size_t)bh, split, max_splits);
}

// ----------------------------------------------------------------- paged pass 1
constexpr int kMaxTableSpan = 72;  // block-table entries one split may touch

template <int G>
__global__ void __launch_bounds__(kThreads)
paged_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ key_cache,
                   const uint16_t* __restrict__ value_cache,
                   const int32_t* __restrict__ block_tables, int table_cols,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
                   int Hq, int Hkv, int num_blocks, int block_size, int bs_log2, int max_len,
                   float scale_log2, int chunk, int max_splits, float* __restrict__ ws_o,
                   float* __restrict__ ws_lse, int32_t* err_flag) {
  constexpr int D = 128;
  constexpr int LPR = D / 8;
  constexpr int U = G >= 4 ? 2 : 4;
  __shared__ int tbl[kMaxTableSpan];
  const int split = blockIdx.x % max_splits;
  const int bg = blockIdx.x / max_splits;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  int toff = 0;
  const int L = paged_len(seq_lens, seq_offset, b, block_size, table_cols, max_len, &toff,
                          err_flag, split == 0 && g == 0 && threadIdx.x == 0);
  const int r0 = split * chunk;
  if (r0 >= L) return;
  const int r1 = min(r0 + chunk, L);
  const int blk0 = r0 >> bs_log2;
  const int nblk = ((r1 - 1) >> bs_log2) - blk0 + 1;
  for (int i = threadIdx.x; i < nblk; i += kThreads) {
    int phys = block_tables[(size_t)b * table_cols + toff + blk0 + i];
    if (phys < 0 || phys >= num_blocks) {
      raise_flag(err_flag, 1);
      phys = -1;
    }
    tbl[i] = phys;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int group = Hq / Hkv;  // == G
  float qr[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 raw = load16(q + ((size_t)b * Hq + (size_t)g * group + j) * D + sub * 8);
    unpack8(raw, qr[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[j][i] *= scale_log2;
  }
  const size_t row_stride = (size_t)Hkv * D;
  const size_t head_off = (size_t)g * D + (size_t)sub * 8;
  const int bs_mask = block_size - 1;
  auto row_at = [&](int t, bool& ok) -> size_t {
    if (!ok) return 0;
    const int phys = tbl[(t >> bs_log2) - blk0];
    if (phys < 0) { ok = false; return 0; }
    return ((size_t)phys * block_size + (t & bs_mask)) * row_stride + head_off;
  };
  HeadState<G> st;
  init_state(st);
  attend_rows<D, G, U>(key_cache, value_cache, qr, r0, r1, wave, lane / LPR, row_at, st);
  merge_groups<LPR, G>(st);
  write_partials<D, G>(st, lane, wave, ws_o, ws_lse, (size_t)b * Hq + (size_t)g * group, split,
                       max_splits);
}

// ------------------------------------------------------------------- pass 2
// Length modes: 0 = static with valid_len (or cap), 1 = paged.
template <int D>
__global__ void __launch_bounds__(D)
merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int heads,
             int chunk, int max_splits, int mode, const int32_t* __restrict__ valid_len, int cap,
             const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
             int block_size, int table_cols, int max_len, float* __restrict__ out,
             float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / heads;
  const int d = threadIdx.x;
  int L;
  if (mode == 0) {
    L = static_len(valid_len, b, cap, nullptr, false);
  } else {
    int toff;
    L = paged_len(seq_lens, seq_offset, b, block_size, table_cols, max_len, &toff, nullptr,
                  false);
  }
  const int n = (L + chunk - 1) / chunk;
  const float* lp = ws_lse + (size_t)bh * max_splits;
  const float* op = ws_o + (size_t)bh * max_splits * D + d;
  float M = kNegInf;
  for (int j = 0; j < n; ++j) M = fmaxf(M, lp[j]);
  if (M == kNegInf) {
    out[(size_t)bh * D + d] = 0.f;
    if (lse && d == 0) lse[bh] = kNegInf;
    return;
  }
  float num = 0.f, den = 0.f;
  for (int j = 0; j < n; ++j) {
    const float w = exp2_fast(lp[j] - M);
    num += w * op[(size_t)j * D];
    den += w;
  }
  out[(size_t)bh * D + d] = num / den;
  if (lse && d == 0) lse[bh] = (M + __log2f(den)) * kLn2;
}

// ------------------------------------------------------------------- planning
static int round_up(int x, int m) { return (x + m - 1) / m * m; }

SplitPlan plan_static(int B, int H, int cap, int D, int forced_splits) {
  (void)D;
  SplitPlan p;
  if (forced_splits > 0) {
    const int per = (cap + forced_splits - 1) / forced_splits;
    p.chunk = per < kMinChunk ? kMinChunk : round_up(per, kMinChunk);
  } else {
    // about 2048 workgroup slots at full capacity; 64..1024 rows per split
    long long want = ((long long)B * H * cap + 2047) / 2048;
    int c = (int)(want > 1024 ? 1024 : want);
    p.chunk = c < kMinChunk ? kMinChunk : round_up(c, kMinChunk);
  }
  if (cap <= 0) p.chunk = kMinChunk;
  p.max_splits = cap > 0 ? (cap + p.chunk - 1) / p.chunk : 1;
  return p;
}

size_t static_workspace_bytes(int B, int H, int cap, int D) {
  const size_t splits = cap > 0 ? (size_t)(cap + kMinChunk - 1) / kMinChunk : 1;
  return (size_t)B * H * splits * (size_t)(D + 1) * sizeof(float);
}

hipError_t launch_decode_static(const float* q, const void* k_cache, const void* v_cache,
                                const int32_t* mask, const int32_t* valid_len, int B, int H,
                                int cap, int D, float scale, float* out, float* lse, void* ws,
                                const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o + (size_t)B * H * plan.max_splits * D;
  const float scale_log2 = scale * kLog2e;
  const dim3 grid1((unsigned)(B * H * plan.max_splits));
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  if (D == 128) {
    hipLaunchKernelGGL(static_split_kernel<128>, grid1, dim3(kThreads), 0, stream, q, kc, vc,
                       mask, valid_len, H, cap, scale_log2, plan.chunk, plan.max_splits, ws_o,
                       ws_lse, err_flag);
    hipLaunchKernelGGL(merge_kernel<128>, dim3(B * H), dim3(128), 0, stream, ws_o, ws_lse, H,
                       plan.chunk, plan.max_splits, 0, valid_len, cap, nullptr, nullptr, 1, 0, 0,
                       out, lse);
  } else {
    hipLaunchKernelGGL(static_split_kernel<64>, grid1, dim3(kThreads), 0, stream, q, kc, vc,
                       mask, valid_len, H, cap, scale_log2, plan.chunk, plan.max_splits, ws_o,
                       ws_lse, err_flag);
    hipLaunchKernelGGL(merge_kernel<64>, dim3(B * H), dim3(64), 0, stream, ws_o, ws_lse, H,
                       plan.chunk, plan.max_splits, 0, valid_len, cap, nullptr, nullptr, 1, 0, 0,
                       out, lse);
  }
  return hipGetLastError();
}

SplitPlan plan_paged(int B, int Hkv, int max_seq_len, int block_size, int forced_splits) {
  SplitPlan p;
  const int unit = block_size > kMinChunk ? block_size : kMinChunk;
  // one split may touch at most kMaxTableSpan - 1 blocks
  const int most = ((kMaxTableSpan - 2) * block_size) / unit * unit;
  int c;
  if (forced_splits > 0) {
    c = round_up((max_seq_len + forced_splits - 1) / forced_splits, unit);
  } else {
    long long want = ((long long)B * Hkv * max_seq_len + 2047) / 2048;
    c = (int)(want > 512 ? 512 : want);
    c = round_up(c < 1 ? 1 : c, unit);
  }
  if (c < unit) c = unit;
  if (c > most) c = most;
  p.chunk = c;
  p.max_splits = max_seq_len > 0 ? (max_seq_len + c - 1) / c : 1;
  return p;
}

size_t paged_workspace_bytes(int B, int Hq, int D, int max_seq_len, int block_size) {
  const int unit = block_size > kMinChunk ? block_size : kMinChunk;
  const size_t splits = max_seq_len > 0 ? (size_t)(max_seq_len + unit - 1) / unit : 1;
  return (size_t)B * Hq * splits * (size_t)(D + 1) * sizeof(float);
}

hipError_t launch_decode_paged(const void* q, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse, void* ws,
                               const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  (void)D;
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o + (size_t)B * Hq * plan.max_splits * 128;
  const float scale_log2 = scale * kLog2e;
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const dim3 grid1((unsigned)(B * Hkv * plan.max_splits));
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(key_cache);
  const auto* vc = static_cast<const uint16_t*>(value_cache);
  const int G = Hq / Hkv;
#define DAKV_PAGED(GG)                                                                        \
  hipLaunchKernelGGL(paged_split_kernel<GG>, grid1, dim3(kThreads), 0, stream, qb, kc, vc,   \
                     block_tables, table_cols, seq_lens, seq_offset, Hq, Hkv, num_blocks,    \
                     block_size, bs_log2, max_seq_len, scale_log2, plan.chunk,               \
                     plan.max_splits, ws_o, ws_lse, err_flag)
  switch (G) {
    case 1: DAKV_PAGED(1); break;
    case 2: DAKV_PAGED(2); break;
    case 4: DAKV_PAGED(4); break;
    case 8: DAKV_PAGED(8); break;
    default: return hipErrorInvalidValue;
  }
#undef DAKV_PAGED
  hipLaunchKernelGGL(merge_kernel<128>, dim3(B * Hq), dim3(128), 0, stream, ws_o, ws_lse, Hq,
                     plan.chunk, plan.max_splits, 1, nullptr, 0, seq_lens, seq_offset, block_size,
                     table_cols, max_seq_len, out, lse);
  return hipGetLastError();
}

}  // namespace dakv
