// Top-k sparse MLA-style decode on the matrix cores (FlashMLA on Huawei Ascend,
// "Mathematical formulation" and "Course of computation"): all query heads of a
// sequence share the gathered latent rows G = kv[b][indices[b]] (d_qk = 576), the
// value is G[:, :512], and the softmax runs online over blocks of the index list
// with a running max that is only moved when it grows by more than a threshold
// ("skip scale").
//
// Work split: one workgroup (4 waves) per (sequence, 64 query heads, 256 indices).
// Each wave owns 16 heads.  Per tile of 32 gathered rows:
//   * the rows are fetched from HBM (16-byte loads, issued one tile ahead) into
//     an LDS buffer (row pitch 1168 bytes to spread banks), double-buffered;
//   * S^T[token, head] = G Q^T with v_mfma_f32_16x16x32_bf16: A = 16 rows x 32
//     dims and B = Q^T (the group's Q rows, staged in LDS once per split) both
//     read from LDS, six k-steps of operands ahead of their MFMAs;
//   * the C layout of S^T puts head (lane % 16) and 4 tokens per half-tile in each
//     lane, which is already the A layout of P for O = P V when the 8 tokens of a
//     lane group are taken in the order {4g..4g+3, 16+4g..16+4g+3};
//   * P enters the matrix core as bf16 hi + lo parts (two MFMAs per block);
//   * V (the first 512 dims of the same rows) is read from LDS as 8 rows x 16
//     bytes per lane and transposed in registers into the B operand (8 tokens of
//     one dim per MFMA), so no transposing LDS access is needed; output column n
//     of MFMA j is dim 8n + j of the 128-dim block.
// Each split writes o / l and the log2-sum-exp; a merge kernel combines splits.
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
constexpr int kTile = 32;                               // gathered rows per tile
constexpr int kSplit = 256;                             // indices per workgroup
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 64;
constexpr int kChunksPerRow = kRowBytes / 16;           // 72
constexpr int kLoads = kTile * kChunksPerRow / 256;     // 9 per thread per tile
constexpr int kKSteps = kDqk / 32;                      // 18
constexpr int kVBlocks = kDv / 128;                     // 4
// The page's rescale threshold is 6 in natural-log units; scores here are in log2.
constexpr float kRescale = 6.0f * kLog2e;
constexpr uint32_t kNoRow = 0x80000000u;  // a buffer offset past any sequence: loads 0

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__global__ void __launch_bounds__(256)
sparse_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const int32_t* __restrict__ indices, int B, int Hq, int s_kv, int topk,
                    float scale_log2, int n_hg, int n_splits, int per_hg,
                    float* __restrict__ ws_o, float* __restrict__ ws_lse, int32_t* err_flag) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t qs[kHeadsPerWG * kPitch];  // this group's Q rows
  __shared__ uint32_t rows[kSplit];  // byte offset of each index's row in kv[b], or kNoRow
  // blockIdx -> (head group, unit); units of the same (b, split) in different head
  // groups are per_hg (a multiple of 8) apart, so they land on the same XCD.
  const int hg = blockIdx.x / per_hg;
  const int u = blockIdx.x - hg * per_hg;
  if (u >= B * n_splits) return;
  const int b = u / n_splits;
  const int split = u - b * n_splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;   // lane group 0..3
  const int col16 = lane & 15;
  const int t0 = split * kSplit;
  const int ntok = min(kSplit, topk - t0);
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

  u32x4_t stage[kLoads];
  auto load_tile = [&](int ti) {
    uint32_t off[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + 256 * k;
      const int r = c / kChunksPerRow;
      const uint32_t o = rows[ti * kTile + r];
      off[k] = o == kNoRow ? kNoRow : o + (uint32_t)(c - r * kChunksPerRow) * 16;
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k)
      stage[k] = __builtin_amdgcn_raw_buffer_load_b128(kvr, (int)off[k], 0, 0);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + 256 * k;
      const int r = c / kChunksPerRow;
      const int col = c - r * kChunksPerRow;
      *reinterpret_cast<u32x4_t*>(&tile[buf][r * kPitch + col * 16]) = stage[k];
    }
  };

  const int head0 = hg * kHeadsPerWG + wave * kHeadsPerWave;
  const bool active = head0 < Hq;
  // This group's 64 query rows go to LDS (rows past Hq read as zeros); a wave
  // reads the B operand Q^T of its 16 heads from there: lane -> head head0 +
  // col16, dims 8*grp + 32*s .. +8.
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + (size_t)b * Hq * kDqk, (short)0, Hq * kRowBytes, 0x00020000);
    constexpr int kQLoads = kHeadsPerWG * kChunksPerRow / 256;  // 18
    const int hbase = hg * kHeadsPerWG;
#pragma unroll
    for (int k = 0; k < kQLoads; ++k) {
      const int c = tid + 256 * k;
      const int r = c / kChunksPerRow;
      const int col = c - r * kChunksPerRow;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          qr, (int)((uint32_t)(hbase + r) * kRowBytes + col * 16), 0, 0);
      *reinterpret_cast<u32x4_t*>(&qs[r * kPitch + col * 16]) = v;
    }
  }
  const uint8_t* qrow = qs + (wave * kHeadsPerWave + col16) * kPitch + grp * 16;
  f32x4_t oacc[kVBlocks * 8];
#pragma unroll
  for (int j = 0; j < kVBlocks * 8; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // running max used for the exponentials, head head0 + col16
  float lsum = 0.f;       // this lane's share of the sum of exponentials

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(it + 1);
    if (active) {
      const uint8_t* T = tile[buf];
      // S^T = G Q^T: the A operands of 6 k-steps of both halves are read from LDS
      // together, then their 12 MFMAs run
      f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      const uint8_t* arow0 = T + col16 * kPitch + grp * 16;
      const uint8_t* arow1 = arow0 + 16 * kPitch;
#pragma unroll
      for (int s0 = 0; s0 < kKSteps; s0 += 6) {
        u32x4_t a0[6], a1[6], qv[6];
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          a0[k] = *reinterpret_cast<const u32x4_t*>(arow0 + (s0 + k) * 64);
          a1[k] = *reinterpret_cast<const u32x4_t*>(arow1 + (s0 + k) * 64);
          qv[k] = *reinterpret_cast<const u32x4_t*>(qrow + (s0 + k) * 64);
        }
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          const bf16x8_t qk = as_bf16x8(qv[k]);
          st[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[k]), qk, st[0], 0, 0, 0);
          st[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[k]), qk, st[1], 0, 0, 0);
        }
      }
      // st[h][i] = score of token 16h + 4*grp + i (of this tile) for head col16
      float sc[8];
      float tmax = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = it * kTile + 16 * h + 4 * grp + i;
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
      // O += P V, four blocks of 128 dims; block c+1's rows are read from LDS
      // before block c's MFMAs
      u32x4_t R[2][8];
      auto read_block = [&](int c, u32x4_t (&dst)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int trow = (i < 4) ? (4 * grp + i) : (16 + 4 * grp + (i - 4));
          dst[i] = *reinterpret_cast<const u32x4_t*>(T + trow * kPitch + (c * 128 + col16 * 8) * 2);
        }
      };
      read_block(0, R[0]);
#pragma unroll
      for (int c = 0; c < kVBlocks; ++c) {
        if (c + 1 < kVBlocks) read_block(c + 1, R[(c + 1) & 1]);
        const u32x4_t (&Rc)[8] = R[c & 1];
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
    }
    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: per head, total of the exponentials over the 4 lane groups.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float lh[4], mh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lh[i] = __shfl(lsum, 4 * grp + i);
    mh[i] = __shfl(m_ref, 4 * grp + i);
  }
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = head0 + 4 * grp + i;
    const size_t unit = ((size_t)b * Hq + head) * n_splits + split;
    float* dst = ws_o + unit * kDv + col16 * 8;
    const bool empty = mh[i] == kNegInf;
    const float inv = empty ? 0.f : 1.f / lh[i];
#pragma unroll
    for (int c = 0; c < kVBlocks; ++c) {
      float4 lo4, hi4;
      lo4.x = oacc[c * 8 + 0][i] * inv; lo4.y = oacc[c * 8 + 1][i] * inv;
      lo4.z = oacc[c * 8 + 2][i] * inv; lo4.w = oacc[c * 8 + 3][i] * inv;
      hi4.x = oacc[c * 8 + 4][i] * inv; hi4.y = oacc[c * 8 + 5][i] * inv;
      hi4.z = oacc[c * 8 + 6][i] * inv; hi4.w = oacc[c * 8 + 7][i] * inv;
      *reinterpret_cast<float4*>(dst + c * 128) = lo4;
      *reinterpret_cast<float4*>(dst + c * 128 + 4) = hi4;
    }
    if (col16 == 0) ws_lse[unit] = empty ? kNegInf : mh[i] + __log2f(lh[i]);
  }
}

// Combine the splits of one (sequence, head): weights 2^(lse_j - max).
__global__ void __launch_bounds__(256)
sparse_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    int n_splits, float* __restrict__ out, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* lp = ws_lse + (size_t)bh * n_splits;
  float M = kNegInf;
  for (int j = 0; j < n_splits; ++j) M = fmaxf(M, lp[j]);
  for (int d = threadIdx.x; d < kDv; d += 256) {
    if (M == kNegInf) {
      out[(size_t)bh * kDv + d] = 0.f;
      continue;
    }
    float num = 0.f, den = 0.f;
    for (int j = 0; j < n_splits; ++j) {
      const float w = exp2_fast(lp[j] - M);
      num += w * ws_o[((size_t)bh * n_splits + j) * kDv + d];
      den += w;
    }
    out[(size_t)bh * kDv + d] = num / den;
  }
  if (lse && threadIdx.x == 0) {
    if (M == kNegInf) {
      lse[bh] = kNegInf;
    } else {
      float den = 0.f;
      for (int j = 0; j < n_splits; ++j) den += exp2_fast(lp[j] - M);
      lse[bh] = (M + __log2f(den)) * kLn2;
    }
  }
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
