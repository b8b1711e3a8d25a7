// Top-k sparse MLA-style decode on the matrix cores (FlashMLA on Huawei Ascend,
// "Mathematical formulation" and "Course of computation"): all query heads of a
// sequence share the gathered latent rows G = kv[b][indices[b]] (d_qk = 576), the
// value is G[:, :512], and the softmax runs online over blocks of the index list
// with a running max that is only moved when it grows by more than a threshold
// ("skip scale").
//
// Work split: one workgroup (4 waves) per (sequence, 32 query heads, 512
// indices); the head groups of one (sequence, index split) sit a multiple of 8
// workgroups apart, so they run on one XCD and share its L2.  Wave w owns 16
// heads (head block w & 1) and one half of every 64-row tile (rows 32 (w >> 1)
// .. +32).  Per tile:
//   * the 64 gathered rows are fetched from HBM (16-byte loads into registers,
//     one tile ahead, in two halves) and stored to an LDS buffer (row pitch 1168
//     bytes to spread banks), double-buffered; both head blocks read a row there;
//   * S^T[token, head] = G Q^T with v_mfma_f32_16x16x32_bf16: A = 16 rows x 32
//     dims from LDS, B = Q^T of the wave's 16 heads, held in registers for the
//     whole split (18 k-steps x 16 bytes per lane);
//   * the C layout of S^T puts head (lane % 16) and 4 tokens per 16-row half in
//     each lane, which is already the A layout of P for O = P V when the 8 tokens
//     of a lane group are taken in the order {4g..4g+3, 16+4g..16+4g+3};
//   * P enters the matrix core as bf16 hi + lo parts (two MFMAs per block);
//   * V (the first 512 dims of the same rows) is read from LDS as 8 rows x 16
//     bytes per lane and transposed in registers into the B operand (8 tokens of
//     one dim per MFMA); output column n of MFMA j is dim 8n + j of a 128-dim block.
// At the end the two row-half waves of a head block merge through LDS, and the
// split writes o / l and the log2-sum-exp; a merge kernel combines the splits.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;                     // 1152
constexpr int kPitch = kRowBytes + 16;                  // LDS row pitch
constexpr int kTile = 64;                               // gathered rows per tile
constexpr int kHalf = kTile / 2;                        // rows of a tile one wave takes
constexpr int kSplit = 512;                             // indices per workgroup
constexpr int kTiles = kSplit / kTile;                  // 8
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 32;
constexpr int kChunksPerRow = kRowBytes / 16;           // 72
constexpr int kLoads = kTile * kChunksPerRow / 256;     // 18 per thread per tile
static_assert(kTile * 4 == 256 && kLoads * 4 == kChunksPerRow, "4 threads per tile row");
constexpr int kKSteps = kDqk / 32;                      // 18
constexpr int kVBlocks = kDv / 128;                     // 4
// The page's rescale threshold is 6 in natural-log units; scores here are in log2.
constexpr float kRescale = 6.0f * kLog2e;
constexpr uint32_t kNoRow = 0x80000000u;  // a buffer offset past any sequence: loads 0
static_assert(kTile * kChunksPerRow % 256 == 0, "whole loads per thread");
static_assert(kSplit % kTile == 0, "whole tiles per split");

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__global__ void __launch_bounds__(256)
sparse_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const int32_t* __restrict__ indices, int B, int Hq, int s_kv, int topk,
                    float scale_log2, int n_hg, int n_splits, int per_hg,
                    float* __restrict__ ws_o, float* __restrict__ ws_lse, int32_t* err_flag) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTile * kPitch];
  __shared__ uint32_t rows[kSplit];  // byte offset of each index's row in kv[b], or kNoRow
  const int hg = blockIdx.x / per_hg;
  const int u = blockIdx.x - hg * per_hg;
  if (u >= B * n_splits) return;
  const int b = u / n_splits;
  const int split = u - b * n_splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave & 1;     // head block of the group
  const int th = wave >> 1;    // row half of every tile
  const int grp = lane >> 4;   // lane group 0..3
  const int col16 = lane & 15;
  const int head0 = hg * kHeadsPerWG + hb * kHeadsPerWave;
  const bool active = head0 < Hq;
  const int t0 = split * kSplit;
  const int ntok = min(kSplit, topk - t0);
  // Q^T of the wave's heads as B operands: lane -> head head0 + col16, dims
  // 32 s + 8 grp .. +8 (heads past Hq read as zeros).
  u32x4_t qreg[kKSteps];
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + (size_t)b * Hq * kDqk, (short)0, Hq * kRowBytes, 0x00020000);
    const uint32_t base = (uint32_t)(head0 + col16) * kRowBytes + grp * 16;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      qreg[s] = __builtin_amdgcn_raw_buffer_load_b128(qr, (int)(base + s * 64), 0, 0);
  }
  for (int i = tid; i < kSplit; i += 256) {
    uint32_t r = kNoRow;
    if (i < ntok) {
      const int idx = indices[(size_t)b * topk + t0 + i];
      if (idx >= 0 && idx < s_kv) r = (uint32_t)idx * kRowBytes;
      else raise_flag(err_flag, 4);
    }
    rows[i] = r;
  }
  __syncthreads();
  // the sequence's latent rows as a buffer: an absent row reads as zeros
  const __amdgpu_buffer_rsrc_t kvr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kv) + (size_t)b * s_kv * kDqk, (short)0, (int)(s_kv * kRowBytes),
      0x00020000);
  const int ntiles = (ntok + kTile - 1) / kTile;

  // Register staging of the gathered rows, in two halves of kLoads / 2 loads per
  // thread: while tile it is computed from one LDS buffer, the first half of tile
  // it + 1 is in flight during the scores and goes to the other buffer after them,
  // and the second half is in flight during O += P V and goes there after it.  The
  // tile loop is fully unrolled (straight-line code), so each LDS store waits for
  // exactly its own loads; tiles past the split's end load kNoRow offsets (zeros,
  // no memory traffic).
  // Thread t copies row t / 4 of a tile: 16-byte pieces (t % 4) + 4 k, k < 18,
  // i.e. 64 contiguous bytes per row per load instruction across 4 lanes.
  constexpr int kHalfLoads = kLoads / 2;
  const int my_row = tid >> 2;
  const uint32_t my_piece = (uint32_t)(tid & 3) * 16;
  uint8_t* const lds_dst = &tile[0][my_row * kPitch + my_piece];
  constexpr int kBufBytes = kTile * kPitch;
  u32x4_t stage[kHalfLoads];
  auto load_half = [&](int ti, int part) {
    const uint32_t o = rows[ti * kTile + my_row];
    const uint32_t base = o == kNoRow ? kNoRow : o + my_piece;
#pragma unroll
    for (int k = 0; k < kHalfLoads; ++k) {
      const int kk = part * kHalfLoads + k;
      // past the resource (kNoRow) the load returns zeros with no memory traffic
      stage[k] = __builtin_amdgcn_raw_buffer_load_b128(kvr, (int)(base + (o == kNoRow ? 0u : kk * 64u)), 0, 0);
    }
  };
  auto store_half = [&](int buf, int part) {
#pragma unroll
    for (int k = 0; k < kHalfLoads; ++k) {
      const int kk = part * kHalfLoads + k;
      *reinterpret_cast<u32x4_t*>(lds_dst + buf * kBufBytes + kk * 64) = stage[k];
    }
  };

  f32x4_t oacc[kVBlocks * 8];
#pragma unroll
  for (int j = 0; j < kVBlocks * 8; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // running max used for the exponentials, head head0 + col16
  float lsum = 0.f;       // this lane's share of the sum of exponentials

  load_half(0, 0);
  store_half(0, 0);
  load_half(0, 1);
  store_half(0, 1);
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kTiles; ++it) {
    const int buf = it & 1;
    const bool next = it + 1 < kTiles;
    if (next) load_half(it + 1, 0);
    if (active && it < ntiles) {
      const uint8_t* T = tile[buf] + th * kHalf * kPitch;
      // S^T = G Q^T: the A operands of kBatch k-steps of both 16-row halves are
      // read from LDS together, then their 2 kBatch MFMAs run
      constexpr int kBatch = 3;
      f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      const uint8_t* arow0 = T + col16 * kPitch + grp * 16;
      const uint8_t* arow1 = arow0 + 16 * kPitch;
#pragma unroll
      for (int s0 = 0; s0 < kKSteps; s0 += kBatch) {
        u32x4_t a0[kBatch], a1[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          a0[k] = *reinterpret_cast<const u32x4_t*>(arow0 + (s0 + k) * 64);
          a1[k] = *reinterpret_cast<const u32x4_t*>(arow1 + (s0 + k) * 64);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const bf16x8_t qk = as_bf16x8(qreg[s0 + k]);
          st[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[k]), qk, st[0], 0, 0, 0);
          st[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[k]), qk, st[1], 0, 0, 0);
        }
      }
      // st[h][i] = score of row 16h + 4*grp + i (of this wave's half) for head col16
      float sc[8];
      float tmax = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = it * kTile + th * kHalf + 16 * h + 4 * grp + i;
          const float v = rows[tok] != kNoRow ? st[h][i] * scale_log2 : kNegInf;
          sc[4 * h + i] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(m_ref, tmax);
      if (__any(mnew > m_ref + kRescale)) {
        const float alpha = mnew == kNegInf ? 1.f : exp2_fast(m_ref - mnew);
        lsum *= alpha;
        m_ref = mnew;
        float a4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int j = 0; j < kVBlocks * 8; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[j][i] *= a4[i];
        }
      }
      const float mu = m_ref == kNegInf ? 0.f : m_ref;
      if (next) {
        store_half(buf ^ 1, 0);
        load_half(it + 1, 1);
      }
      // P as two bf16 parts (p = hi + lo to about 16 significant bits): rounding
      // P to one bf16 alone can put the output off by more than 2e-3 when a few
      // rows dominate the softmax.
      bf16x8_t pa, pl;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = exp2_fast(sc[k] - mu);
        lsum += p;
        const __bf16 hi = (__bf16)p;
        pa[k] = hi;
        pl[k] = (__bf16)(p - (float)hi);
      }
      // O += P V, four blocks of 128 dims
#pragma unroll
      for (int c = 0; c < kVBlocks; ++c) {
        u32x4_t Rc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int trow = (i < 4) ? (4 * grp + i) : (16 + 4 * grp + (i - 4));
          Rc[i] = *reinterpret_cast<const u32x4_t*>(T + trow * kPitch + (c * 128 + col16 * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4_t vb;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t lo = Rc[2 * k][j >> 1];
            const uint32_t hi = Rc[2 * k + 1][j >> 1];
            vb[k] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          const bf16x8_t vbf = as_bf16x8(vb);
          oacc[c * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vbf, oacc[c * 8 + j], 0, 0, 0);
          oacc[c * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vbf, oacc[c * 8 + j], 0, 0, 0);
        }
      }
    } else if (next) {
      store_half(buf ^ 1, 0);
      load_half(it + 1, 1);
    }
    if (next) {
      store_half(buf ^ 1, 1);
      __syncthreads();
    }
  }

  // Epilogue.  Per head (lane group g holds heads 4g + i of the block): the
  // wave's max and total of the exponentials.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float lh[4], mh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lh[i] = __shfl(lsum, 4 * grp + i);
    mh[i] = __shfl(m_ref, 4 * grp + i);
  }
  // The row-half-1 wave of each head block hands its state to the row-half-0
  // wave through LDS (tile buffer 0, free once every wave is past the last tile).
  constexpr int kXfer = kVBlocks * 8 * 64 * 4 + 64 * 8;  // floats per head block
  static_assert(2 * kXfer * 4 <= kTile * kPitch, "hand-over fits one tile buffer");
  float* xf = reinterpret_cast<float*>(tile[0]) + hb * kXfer;
  __syncthreads();
  if (th == 1) {
#pragma unroll
    for (int j = 0; j < kVBlocks * 8; ++j)
      *reinterpret_cast<f32x4_t*>(xf + (j * 64 + lane) * 4) = oacc[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[kVBlocks * 8 * 256 + lane * 8 + i] = mh[i];
      xf[kVBlocks * 8 * 256 + lane * 8 + 4 + i] = lh[i];
    }
  }
  __syncthreads();
  if (th == 1 || !active) return;
  float wa[4], wb[4], inv[4], lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mb = xf[kVBlocks * 8 * 256 + lane * 8 + i];
    const float lb = xf[kVBlocks * 8 * 256 + lane * 8 + 4 + i];
    const float M = fmaxf(mh[i], mb);
    if (M == kNegInf) {
      wa[i] = wb[i] = inv[i] = 0.f;
      lse2[i] = kNegInf;
    } else {
      wa[i] = exp2_fast(mh[i] - M);
      wb[i] = exp2_fast(mb - M);
      const float l = lh[i] * wa[i] + lb * wb[i];
      inv[i] = 1.f / l;
      lse2[i] = M + __log2f(l);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = head0 + 4 * grp + i;
    const size_t unit = ((size_t)b * Hq + head) * n_splits + split;
    float* dst = ws_o + unit * kDv + col16 * 8;
    float o[kVBlocks * 8];
#pragma unroll
    for (int j = 0; j < kVBlocks * 8; ++j)
      o[j] = (oacc[j][i] * wa[i] + xf[(j * 64 + lane) * 4 + i] * wb[i]) * inv[i];
#pragma unroll
    for (int c = 0; c < kVBlocks; ++c) {
      *reinterpret_cast<float4*>(dst + c * 128) =
          make_float4(o[c * 8 + 0], o[c * 8 + 1], o[c * 8 + 2], o[c * 8 + 3]);
      *reinterpret_cast<float4*>(dst + c * 128 + 4) =
          make_float4(o[c * 8 + 4], o[c * 8 + 5], o[c * 8 + 6], o[c * 8 + 7]);
    }
    if (col16 == 0) ws_lse[unit] = lse2[i];
  }
}

// Combine the splits of one (sequence, head): weights 2^(lse_j - max).  Splits
// are taken 8 at a time with all 8 loads of a thread issued before their use.
constexpr int kMergeBatch = 8;
static_assert(kDv == 2 * 256, "two columns per thread");

__global__ void __launch_bounds__(256)
sparse_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    int n_splits, float* __restrict__ out, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* lp = ws_lse + (size_t)bh * n_splits;
  const float* op = ws_o + (size_t)bh * n_splits * kDv;
  float M = kNegInf;
  for (int j0 = 0; j0 < n_splits; j0 += kMergeBatch) {
    float x[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) x[k] = j0 + k < n_splits ? lp[j0 + k] : kNegInf;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) M = fmaxf(M, x[k]);
  }
  const int d0 = threadIdx.x * 2;  // two adjacent columns per thread
  float num0 = 0.f, num1 = 0.f, den = 0.f;
  if (M != kNegInf) {
    for (int j0 = 0; j0 < n_splits; j0 += kMergeBatch) {
      float w[kMergeBatch];
      float2 v[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const bool in = j0 + k < n_splits;
        w[k] = in ? lp[j0 + k] : kNegInf;
        v[k] = in ? *reinterpret_cast<const float2*>(op + (size_t)(j0 + k) * kDv + d0)
                  : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const float wk = exp2_fast(w[k] - M);
        num0 += wk * v[k].x;
        num1 += wk * v[k].y;
        den += wk;
      }
    }
  }
  const float inv = M == kNegInf ? 0.f : 1.f / den;
  *reinterpret_cast<float2*>(out + (size_t)bh * kDv + d0) = make_float2(num0 * inv, num1 * inv);
  if (lse && threadIdx.x == 0) lse[bh] = M == kNegInf ? kNegInf : (M + __log2f(den)) * kLn2;
}

static int sparse_splits(int topk) { return (topk + kSplit - 1) / kSplit; }

size_t sparse_workspace_bytes(int B, int Hq, int d_qk, int d_v, int topk) {
  (void)d_qk;
  return (size_t)B * Hq * sparse_splits(topk) * (size_t)(d_v + 1) * sizeof(float);
}

hipError_t launch_sparse(const void* q, const void* kv, const int32_t* indices, int B, int Hq,
                         int s_kv, int d_qk, int d_v, int topk, float sm_scale, float* out,
                         float* lse, void* ws, int32_t* err_flag, hipStream_t stream) {
  (void)d_qk;
  (void)d_v;
  const int n_splits = sparse_splits(topk);
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o + (size_t)B * Hq * n_splits * kDv;
  if (n_splits > 0) {
    const int n_hg = (Hq + kHeadsPerWG - 1) / kHeadsPerWG;
    const int per_hg = (B * n_splits + 7) / 8 * 8;
    hipLaunchKernelGGL(sparse_split_kernel, dim3(n_hg * per_hg), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv),
                       indices, B, Hq, s_kv, topk, sm_scale * kLog2e, n_hg, n_splits, per_hg,
                       ws_o, ws_lse, err_flag);
  }
  hipLaunchKernelGGL(sparse_merge_kernel, dim3(B * Hq), dim3(256), 0, stream, ws_o, ws_lse,
                     n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace dakv
