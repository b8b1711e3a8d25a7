// Split-pass building blocks shared by the decode kernels (bf16 and FP8 caches):
// launch shape, online-softmax state and its in-wave merge, the branch-free row
// loaders, the workspace of split partials, the log-sum-exp merge of one head,
// and the end of a split (waves combined through LDS, then the output or the
// split's partial written).  Every multiply-add here is an explicit fmaf, so that
// each kernel instantiation rounds alike whatever the compiler would contract
// (the fused append + attend step is bit-identical to the two separate calls).
#pragma once

#include "device.hpp"
#include "launch.hpp"

namespace dakv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMinChunk = 64;
constexpr int kMaxSplits = 256;  // splits one unit may have (merge state lives in LDS)

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

// Effective row count of a paged sequence from its cumulative lengths [start,
// end) and table offset: the difference, cut at max_len and at the table's last
// column (toff = the offset in blocks); *bad tells whether anything was cut.
__device__ __forceinline__ int paged_len_of(int start, int end, int off, int block_size,
                                            int table_cols, int max_len, int* toff, bool* bad) {
  int L = end - start;
  *bad = false;
  if (L < 0) { L = 0; *bad = true; }
  if (off < 0 || off % block_size != 0) { L = 0; *bad = true; *toff = 0; }
  else *toff = off / block_size;
  const int room = (table_cols - *toff) * block_size;
  if (L > room) { L = room > 0 ? room : 0; *bad = true; }
  if (L > max_len) { L = max_len; *bad = true; }
  return L;
}

// The same, loading the sequence's entries; inconsistencies are flagged.
__device__ __forceinline__ int paged_len(const int32_t* seq_lens, const int32_t* seq_offset,
                                         int b, int block_size, int table_cols, int max_len,
                                         int* toff, int32_t* err_flag, bool report) {
  bool bad;
  const int L = paged_len_of(seq_lens[b], seq_lens[b + 1], seq_offset ? seq_offset[b] : 0,
                             block_size, table_cols, max_len, toff, &bad);
  if (bad && report) raise_flag(err_flag, 8);
  return L;
}

// Online-softmax state of G query heads for one row group (D/E lanes, E output
// dims per lane).
template <int G, int E = 8>
struct HeadState {
  float m[G], l[G], o[G][E];
};

template <int G, int E>
__device__ __forceinline__ void init_state(HeadState<G, E>& st) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) st.o[j][i] = 0.f;
  }
}

// Merge the row groups of one wave (they differ in the lane bits above the group).
template <int LPR, int G, int E>
__device__ __forceinline__ void merge_groups(HeadState<G, E>& st) {
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
      st.l[j] = fmaf(st.l[j], ws, lo * wo);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float oo = __shfl_xor(st.o[j][i], off);
        st.o[j][i] = fmaf(st.o[j][i], ws, oo * wo);
      }
      st.m[j] = M;
    }
  }
}

// Where a loop step's K/V pieces come from.  Both loaders are branch-free: a row
// that must not be used still issues its load, but the load either touches no
// memory (buffer load past the end of the resource returns zeros) or re-reads a
// fixed in-bounds location whose V value is then replaced by zeros.  Such a row
// enters the update with weight 0, and 0 times a NaN or an infinity left in an
// unused slot of the cache would still be NaN, so its V must be exactly zero.
//
// BufferRows: one (sequence, head) region of the static cache; `off` is a byte
// offset inside it, and kNoRow (past num_records) stands for "no row".
// Cache policy of the K/V row loads: every row is read once, so the loads are
// non-temporal (bit 1 of the buffer instruction's cache-policy operand; the
// paged loads below use the non-temporal global form).  Measured: the static
// fused step call drops from 48.8 to 41.9 us at batch 8.
constexpr int kLoadNonTemporal = 2;

struct BufferRows {
  __amdgpu_buffer_rsrc_t k, v;
  static constexpr uint32_t kNoRow = 0x80000000u;
  __device__ BufferRows(const uint16_t* kbase, const uint16_t* vbase, uint32_t bytes)
      : k(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), (short)0, (int)bytes,
                                            0x00020000)),
        v(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase), (short)0, (int)bytes,
                                            0x00020000)) {}
  // (ok is not needed: the "no row" offset already returns zeros)
  __device__ __forceinline__ void load(uint32_t off, bool, uint4& kr, uint4& vr) const {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(k, (int)off, 0, kLoadNonTemporal);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(v, (int)off, 0, kLoadNonTemporal);
    kr = make_uint4(a[0], a[1], a[2], a[3]);
    vr = make_uint4(b[0], b[1], b[2], b[3]);
  }
};

// GlobalRows: the paged pool through 64-bit addresses; `off` is an element offset
// from the pool base (0, an in-bounds location, for rows that are not used: their
// V is zeroed by a select once it arrives; their K only feeds a score that the
// caller replaces by -inf).
struct GlobalRows {
  const uint16_t* k;
  const uint16_t* v;
  __device__ __forceinline__ void load(size_t off, bool ok, uint4& kr, uint4& vr) const {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
    kr = make_uint4(a[0], a[1], a[2], a[3]);
    vr = make_uint4(ok ? b[0] : 0u, ok ? b[1] : 0u, ok ? b[2] : 0u, ok ? b[3] : 0u);
  }
};

// One loop step's loads: U rows per lane group, K and V.  RowAt(t, ok) returns
// the loader offset of row t (or the loader's "no row" value) and clears ok for
// rows that must not be used.
template <int D, int U, typename Rows, typename RowAt>
__device__ __forceinline__ void issue_rows(const Rows& rows, int base, int r1, int wave,
                                           int slot, RowAt& row_at, uint4 (&kr)[U],
                                           uint4 (&vr)[U], bool (&ok)[U]) {
  constexpr int RPW = 64 / (D / 8);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = base + (u * kWaves + wave) * RPW + slot;
    ok[u] = t < r1;
    const auto off = row_at(t, ok[u]);
    rows.load(off, ok[u], kr[u], vr[u]);
  }
}

struct NoPatch {
  __device__ __forceinline__ void operator()(int, uint4&, uint4&) const {}
};

// One loop step's arithmetic: scores of the U rows for each of the G heads, then
// the online-softmax update of (m, l, o).
template <int D, int G, int U>
__device__ __forceinline__ void consume_rows(const float (&q)[G][8], const uint4 (&kr)[U],
                                             const uint4 (&vr)[U], const bool (&ok)[U],
                                             HeadState<G>& st) {
  constexpr int LPR = D / 8;
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
    st.l[j] = fmaf(st.l[j], alpha, psum);
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

// The row loop shared by the static and paged kernels, for exactly kSteps steps
// (rows at or past r1 are cleared by RowAt).  Each step issues all of its 2U loads
// (U rows per lane group, K and V) before using any; the steps are fully unrolled
// with two register sets used in turn, so the loads of step s+1 are in flight
// while step s is computed and, with no loop, the compiler waits on exactly the
// loads each step needs.  q is pre-scaled by scale * log2(e).  Patch(t, kr, vr)
// may replace row t's values when its step is computed (after its loads have
// arrived, so a replacement never makes the issue wait).
template <int D, int G, int U, int kSteps, typename Rows, typename RowAt, typename Patch>
__device__ __forceinline__ void attend_rows_fixed(const Rows& rows, const float (&q)[G][8],
                                                  int r0, int r1, int wave, int slot,
                                                  RowAt row_at, Patch patch, HeadState<G>& st) {
  constexpr int RPW = 64 / (D / 8);
  constexpr int kStep = kWaves * RPW * U;
  uint4 kr[2][U], vr[2][U];
  bool ok[2][U];
  issue_rows<D, U>(rows, r0, r1, wave, slot, row_at, kr[0], vr[0], ok[0]);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s + 1 < kSteps)
      issue_rows<D, U>(rows, r0 + (s + 1) * kStep, r1, wave, slot, row_at,
                       kr[(s + 1) & 1], vr[(s + 1) & 1], ok[(s + 1) & 1]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      patch(r0 + s * kStep + (u * kWaves + wave) * RPW + slot, kr[s & 1][u], vr[s & 1][u]);
    consume_rows<D, G, U>(q, kr[s & 1], vr[s & 1], ok[s & 1], st);
  }
}

// Workspace of one decode call (fp32):
//   o   [units * G][max_splits][D]   normalised partial outputs o / l
//   lse [units * G][max_splits]      log2-sum-exp of each partial (-inf if empty)
struct Workspace {
  float* o;
  float* lse;
};

__host__ __device__ inline size_t ws_floats(size_t heads, int max_splits, int D) {
  return heads * (size_t)max_splits * (size_t)(D + 1);
}

// Log-sum-exp merge of one head's n <= kMaxSplits partials by the whole
// workgroup, in one memory round trip: every thread issues its log2-sum-exp load
// (thread j holds split j) together with its first kMergePre partial loads (the
// D/4 float4 columns are shared among kThreads / (D/4) split groups); the max and
// the weights 2^(lse_j - max) go through LDS, and the groups are summed there.
constexpr int kMergePre = 8;

template <int D>
__device__ __forceinline__ void merge_head(const float* __restrict__ lp,
                                           const float* __restrict__ op, int n,
                                           float* __restrict__ outp, float* __restrict__ lsep) {
  static_assert(kMaxSplits <= kThreads, "one split per thread");
  constexpr int kCols = D / 4;
  constexpr int kGroups = kThreads / kCols;
  __shared__ float sm_w[kMaxSplits];
  __shared__ float sm_part[2][kWaves];
  __shared__ float4 sm_red[kThreads];
  const int tid = threadIdx.x;
  const int c = tid % kCols;
  const int grp = tid / kCols;
  const float* cp = op + c * 4;
  const float x = tid < n ? lp[tid] : kNegInf;
  float4 pre[kMergePre];
#pragma unroll
  for (int k = 0; k < kMergePre; ++k) {
    const int j = grp + k * kGroups;
    pre[k] = j < n ? *reinterpret_cast<const float4*>(cp + (size_t)j * D)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float v = x;
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((tid & 63) == 0) sm_part[0][tid >> 6] = v;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm_part[0][0], sm_part[0][1]), fmaxf(sm_part[0][2], sm_part[0][3]));
  const float w = (tid < n && M != kNegInf) ? exp2_fast(x - M) : 0.f;
  if (tid < kMaxSplits) sm_w[tid] = w;
  float den_part = w;
  for (int off = 32; off > 0; off >>= 1) den_part += __shfl_xor(den_part, off);
  if ((tid & 63) == 0) sm_part[1][tid >> 6] = den_part;
  __syncthreads();
  const float den = sm_part[1][0] + sm_part[1][1] + sm_part[1][2] + sm_part[1][3];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kMergePre; ++k) {
    const int j = grp + k * kGroups;
    const float wj = j < n ? sm_w[j] : 0.f;
    acc.x = fmaf(wj, pre[k].x, acc.x); acc.y = fmaf(wj, pre[k].y, acc.y);
    acc.z = fmaf(wj, pre[k].z, acc.z); acc.w = fmaf(wj, pre[k].w, acc.w);
  }
  // more splits than the prefetch covers: kMergePre partials per thread at a time,
  // all loads of a batch issued before its first use
  for (int j0 = grp + kMergePre * kGroups; j0 < n; j0 += kMergePre * kGroups) {
    float4 y[kMergePre];
#pragma unroll
    for (int k = 0; k < kMergePre; ++k) {
      const int j = j0 + k * kGroups;
      y[k] = j < n ? *reinterpret_cast<const float4*>(cp + (size_t)j * D)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kMergePre; ++k) {
      const int j = j0 + k * kGroups;
      const float wj = j < n ? sm_w[j] : 0.f;
      acc.x = fmaf(wj, y[k].x, acc.x); acc.y = fmaf(wj, y[k].y, acc.y);
      acc.z = fmaf(wj, y[k].z, acc.z); acc.w = fmaf(wj, y[k].w, acc.w);
    }
  }
  sm_red[tid] = acc;
  __syncthreads();
  if (tid < kCols) {
#pragma unroll
    for (int g = 1; g < kGroups; ++g) {
      const float4 y = sm_red[tid + g * kCols];
      acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
    }
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != kNegInf) {
      const float inv = 1.f / den;
      r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    *reinterpret_cast<float4*>(outp + c * 4) = r;
    if (lsep && tid == 0) *lsep = M == kNegInf ? kNegInf : (M + __log2f(den)) * kLn2;
  }
  __syncthreads();
}

// End of a split without the in-wave merge: every lane group's state (kWaves x RPW
// of them, RPW = 64 / (D / E) per wave) goes to LDS at once and each output element
// combines all of them after one barrier.  (The in-wave merge first took two rounds of
// cross-lane exchanges, each waiting on the previous.)
template <int D, int E>
__device__ __forceinline__ void finish_split_flat(const HeadState<1, E>& st, int lane, int wave,
                                                  const Workspace& ws, size_t head0, int split,
                                                  int n, int max_splits, float* __restrict__ out,
                                                  float* __restrict__ lse) {
  constexpr int LPR = D / E;
  constexpr int RPW = 64 / LPR;
  constexpr int NS = kWaves * RPW;  // lane groups of the workgroup
  __shared__ float sm_o[NS][D];
  __shared__ float sm_m[NS];
  __shared__ float sm_l[NS];
  const int g = wave * RPW + lane / LPR;
  const int sub = lane % LPR;
#pragma unroll
  for (int i = 0; i < E; ++i) sm_o[g][sub * E + i] = st.o[0][i];
  if (sub == 0) {
    sm_m[g] = st.m[0];
    sm_l[g] = st.l[0];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NS; ++k) M = fmaxf(M, sm_m[k]);
    float val = 0.f, lse2 = kNegInf;
    if (M != kNegInf) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const float wt = exp2_fast(sm_m[k] - M);
        num = fmaf(wt, sm_o[k][d], num);
        den = fmaf(wt, sm_l[k], den);
      }
      val = num / den;
      lse2 = M + __log2f(den);
    }
    if (n == 1) {
      out[head0 * D + d] = val;
      if (lse && d == 0) lse[head0] = lse2 * kLn2;
    } else {
      const size_t row = head0 * max_splits + split;
      ws.o[row * D + d] = val;
      if (d == 0) ws.lse[row] = lse2;
    }
  }
}

// End of a split: combine the waves through LDS, then write the output directly
// (a sequence that fits one split) or this split's partial for merge_kernel.
// (The splits are not merged in the last one to finish: publishing the partials
// to another XCD takes a device-scope release that writes back the L2, or
// device-coherent atomics; both measured far slower than a second launch.)
template <int D, int G, int E>
__device__ __forceinline__ void finish_split(const HeadState<G, E>& st, int lane, int wave,
                                             const Workspace& ws, size_t head0, int split,
                                             int n, int max_splits, float* __restrict__ out,
                                             float* __restrict__ lse) {
  constexpr int LPR = D / E;
  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int i = 0; i < E; ++i) sm_o[wave][j][lane * E + i] = st.o[j][i];
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
    float val = 0.f, lse2 = kNegInf;
    if (M != kNegInf) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = exp2_fast(sm_m[w][j] - M);
        num = fmaf(wt, sm_o[w][j][d], num);
        den = fmaf(wt, sm_l[w][j], den);
      }
      val = num / den;
      lse2 = M + __log2f(den);
    }
    if (n == 1) {
      out[(head0 + j) * D + d] = val;
      if (lse && d == 0) lse[head0 + j] = lse2 * kLn2;
    } else {
      const size_t row = (head0 + j) * max_splits + split;
      ws.o[row * D + d] = val;
      if (d == 0) ws.lse[row] = lse2;
    }
  }
}

// ------------------------------------------------------------------ paged layout
constexpr int kMaxTableSpan = 72;  // block-table entries one split may touch

// Step shape of the paged kernel per group size G: U rows per lane group per
// step and kSteps steps per unrolled super-step (fewer rows in flight when each
// row feeds more heads and the state takes more registers).
template <int G> struct PagedShape;
template <> struct PagedShape<1> { static constexpr int U = 4, kSteps = 2; };
template <> struct PagedShape<2> { static constexpr int U = 4, kSteps = 2; };
template <> struct PagedShape<4> { static constexpr int U = 2, kSteps = 4; };
template <> struct PagedShape<8> { static constexpr int U = 2, kSteps = 2; };

constexpr int kRowGroups = 16;  // lane groups of 16 lanes in a workgroup (D = 128)
constexpr int kPagedRowsTarget = 4096;  // workgroups of a call, if all were full length

// End of an all-heads split: every group's state goes to LDS, then each output
// element combines the TS groups of its KV head and is written out directly
// (one split) or as this split's partial.
template <int G>
__device__ __forceinline__ void finish_split_rows(const HeadState<G>& st, int gi, int sub, int Hkv,
                                                  int ts, const Workspace& ws, size_t head0,
                                                  int split, int n, int max_splits,
                                                  float* __restrict__ out,
                                                  float* __restrict__ lse) {
  constexpr int D = 128;
  __shared__ float sm_o[kRowGroups][G][D];
  __shared__ float sm_m[kRowGroups][G];
  __shared__ float sm_l[kRowGroups][G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_o[gi][j][sub * 8 + i] = st.o[j][i];
    if (sub == 0) {
      sm_m[gi][j] = st.m[j];
      sm_l[gi][j] = st.l[j];
    }
  }
  __syncthreads();
  const int total = Hkv * G * D;
  for (int idx = threadIdx.x; idx < total; idx += kThreads) {
    const int hj = idx / D;  // query head within the sequence: h * G + j
    const int d = idx - hj * D;
    const int h = hj / G;
    const int j = hj - h * G;
    float M = kNegInf;
    for (int s = 0; s < ts; ++s) M = fmaxf(M, sm_m[h + s * Hkv][j]);
    float val = 0.f, lse2 = kNegInf;
    if (M != kNegInf) {
      float num = 0.f, den = 0.f;
      for (int s = 0; s < ts; ++s) {
        const int g2 = h + s * Hkv;
        const float wt = exp2_fast(sm_m[g2][j] - M);
        num = fmaf(wt, sm_o[g2][j][d], num);
        den = fmaf(wt, sm_l[g2][j], den);
      }
      val = num / den;
      lse2 = M + __log2f(den);
    }
    if (n == 1) {
      out[(head0 + hj) * D + d] = val;
      if (lse && d == 0) lse[head0 + hj] = lse2 * kLn2;
    } else {
      const size_t row = (head0 + hj) * max_splits + split;
      ws.o[row * D + d] = val;
      if (d == 0) ws.lse[row] = lse2;
    }
  }
}

constexpr int kStaticChunkMax = 256;  // rows per split of the static layout, at most

__host__ inline Workspace carve(void* ws, size_t heads, int max_splits, int D) {
  Workspace w;
  w.o = static_cast<float*>(ws);
  w.lse = w.o + heads * (size_t)max_splits * D;
  return w;
}

// merge_kernel over the splits of a paged call (D = 128, lengths from seq_lens).
hipError_t launch_paged_merge(const Workspace& w, int B, int Hq, int chunk, int max_splits,
                              const int32_t* seq_lens, const int32_t* seq_offset,
                              int block_size, int table_cols, int max_seq_len, float* out,
                              float* lse, hipStream_t stream);

// merge_kernel over the splits of a static-layout call (one launch, B * H heads).
hipError_t launch_static_merge(const Workspace& w, int B, int H, int D, int chunk,
                               int max_splits, const int32_t* valid_len, int cap, float* out,
                               float* lse, hipStream_t stream);


}  // namespace dakv
