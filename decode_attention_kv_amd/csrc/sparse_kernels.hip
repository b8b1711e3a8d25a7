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
// heads (head block w & 1) and one 32-row half (w >> 1) of every 64-row tile.
//   * Rows are gathered by direct-to-LDS buffer loads (16 bytes per lane, no
//     registers) into two tile buffers: tile it + 1 is in flight while tile it is
//     computed; one barrier per tile.  A tile is 64 unpadded 1152-byte rows; the
//     16-byte pieces of row r are stored in a permuted order (XOR of the piece's
//     low 3 bits with a function of r) so that both LDS read patterns below hit
//     16 distinct bank groups.
//   * S^T[token, head] = G Q^T with v_mfma_f32_16x16x32_bf16: A = 16 rows x 32
//     dims from LDS (read a batch of k-steps ahead), B = Q^T of the wave's 16
//     heads, held in registers for the whole split (18 k-steps x 16 bytes per
//     lane); four accumulation chains (two 16-row halves x even/odd k-steps).
//   * The C layout of S^T (lane: head lane % 16, tokens 4 (lane / 16) + i of
//     each half) is the A layout of P for O = P V when the 8 tokens of a lane
//     group are taken in the order {4g..4g+3, 16+4g..16+4g+3}; P enters the
//     matrix core as bf16 hi + lo parts (two MFMAs per block).
//   * The B operand of P V (8 rows of one dim per lane) comes straight from LDS
//     with two transposing reads ds_read_b64_tr_b16: lane j of a 16-lane group
//     points at row 4 (group) + j / 4 (+16), dims 4 (j % 4) .. +3 of a 16-dim
//     block, and lane i receives dim i of that block for the 4 rows.
// At the end the two row-half waves of a head block merge through LDS, and the
// split writes o / l and the log2-sum-exp; a merge kernel combines the splits.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;                     // 1152
constexpr int kPieces = kRowBytes / 16;                 // 72 pieces of 16 bytes
constexpr int kTile = 64;                               // gathered rows per tile
constexpr int kHalf = kTile / 2;                        // rows of a tile one wave takes
constexpr int kTileBytes = kTile * kRowBytes;           // 73728
constexpr int kSplit = 512;                             // indices per workgroup
constexpr int kTiles = kSplit / kTile;                  // 8
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 32;
constexpr int kDmaPerWave = kTileBytes / 1024 / 4;      // 18 wave loads of 1 KiB per tile
constexpr int kKSteps = kDqk / 32;                      // 18
constexpr int kDimBlocks = kDv / 16;                    // 32 output blocks of 16 dims
// The page's rescale threshold is 6 in natural-log units; scores here are in log2.
constexpr float kRescale = 6.0f * kLog2e;
constexpr uint32_t kNoRow = 0x80000000u;  // a buffer offset past any sequence: loads 0
static_assert(kTileBytes % 4096 == 0, "whole 1 KiB wave loads per wave");
static_assert(kPieces % 8 == 0, "pieces permute within groups of 8");
static_assert(kSplit % kTile == 0, "whole tiles per split");

// Position of piece p of row r inside the row (an involution: it also maps a
// position back to its piece).
__device__ __forceinline__ int piece_slot(int p, int r) {
  const int k = (r >> 1) & 7;
  const int x = ((k << 1) & 7) | (k >> 2);
  return (p & ~7) | ((p & 7) ^ x);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t join_bf16x4(const i16x4_t& lo, const i16x4_t& hi) {
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

__global__ void __launch_bounds__(256)
sparse_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const int32_t* __restrict__ indices, int B, int s_q, int Hq, int s_kv,
                    int topk, float scale_log2, int n_hg, int n_splits, int per_hg,
                    float* __restrict__ ws_o, float* __restrict__ ws_lse, int32_t* err_flag) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[kTileBytes];
  __shared__ uint32_t rows[kSplit];  // byte offset of each index's row in kv[b], or kNoRow
  uint8_t* const ring[2] = {buf0, buf1};
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
  // the sequence's latent rows as a buffer (the q-tokens of one sequence, b / s_q,
  // share them): an absent row reads as zeros
  const __amdgpu_buffer_rsrc_t kvr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kv) + (size_t)(b / s_q) * s_kv * kDqk, (short)0,
      (int)(s_kv * kRowBytes), 0x00020000);
  const int ntiles = (ntok + kTile - 1) / kTile;

  // Tile ti into a buffer: wave load I (this wave's I = 18 wave + k) fills bytes
  // [1024 I, 1024 I + 1024) of the tile, lane L the 16 bytes at 1024 I + 16 L,
  // i.e. position c = 64 I + L = 72 r + s of row r, which holds piece
  // piece_slot(s, r).  Tiles past the split's end load kNoRow offsets (zeros).
  auto fetch_tile = [&](int ti, uint8_t* dst) {
    uint32_t off[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int I = wave * kDmaPerWave + k;
      const int c = I * 64 + lane;
      const int r = c / kPieces;
      const int p = piece_slot(c - r * kPieces, r);
      const uint32_t o = rows[ti * kTile + r];
      off[k] = o == kNoRow ? kNoRow : o + (uint32_t)p * 16;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int I = wave * kDmaPerWave + k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kvr, (lds_void*)(dst + I * 1024), 16, (int)off[k],
                                               0, 0, 0);
    }
  };
  fetch_tile(0, buf0);
  // Q^T of the wave's heads as B operands, loaded while tile 0 is in flight:
  // lane -> head head0 + col16, dims 32 s + 8 grp .. +8 (heads past Hq read as
  // zeros).
  u32x4_t qreg[kKSteps];
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + (size_t)b * Hq * kDqk, (short)0, Hq * kRowBytes, 0x00020000);
    const uint32_t base = (uint32_t)(head0 + col16) * kRowBytes + grp * 16;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      qreg[s] = __builtin_amdgcn_raw_buffer_load_b128(qr, (int)(base + s * 64), 0, 0);
  }

  f32x4_t oacc[kDimBlocks];
#pragma unroll
  for (int j = 0; j < kDimBlocks; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // running max used for the exponentials, head head0 + col16
  float lsum = 0.f;       // this lane's share of the sum of exponentials

  // A operand of k-step s, half h: row 32 th + 16 h + col16, piece 4 s + grp.
  const int arow0 = th * kHalf + col16;
  const int arow1 = arow0 + 16;
  // transposing reads of 16-dim block jb: rows 32 th + 4 grp + col16 / 4 (+16),
  // dims 16 jb + 4 (col16 % 4) .. +3: piece 2 jb + (col16 % 4) / 2, byte
  // 8 (col16 & 1) of it.
  const int vrow0 = th * kHalf + 4 * grp + (col16 >> 2);
  const int vrow1 = vrow0 + 16;
  const int vsub = (col16 & 3) >> 1;
  const int vhalf = (col16 & 1) * 8;
  // Byte offsets within a row of the pieces these lanes read: the permutation
  // only moves a piece inside its group of 8 (128 bytes), so k-step s reads at
  // 128 (s / 2) + aoff[h][s % 2] and dim block jb at 128 (jb / 4) + voff[r][jb % 4].
  int aoff[2][2], voff[2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    aoff[0][par] = piece_slot(4 * par + grp, arow0) * 16;
    aoff[1][par] = piece_slot(4 * par + grp, arow1) * 16;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    voff[0][j] = piece_slot(2 * j + vsub, vrow0) * 16 + vhalf;
    voff[1][j] = piece_slot(2 * j + vsub, vrow1) * 16 + vhalf;
  }

#pragma unroll
  for (int it = 0; it < kTiles; ++it) {
    // this wave's loads of tile it are complete (none later is in flight yet);
    // the barrier makes every wave's part visible and ends every wave's reads of
    // tile it - 1, whose buffer the next fetch refills
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0) only
    __builtin_amdgcn_s_barrier();
    if (it + 1 < kTiles) fetch_tile(it + 1, ring[(it + 1) & 1]);
    if (active && it < ntiles) {
      const uint8_t* T = ring[it & 1];
      // S^T = G Q^T over 18 k-steps: chains (half, k-step parity); A operands
      // read from LDS a batch of 3 k-steps ahead (scheduling barriers keep it so)
      f32x4_t st[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) st[h][0] = st[h][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // piece 4 s + grp of a row sits at 128 (s / 2) + aoff[h][s % 2]
      const uint8_t* ap0 = T + arow0 * kRowBytes;
      const uint8_t* ap1 = T + arow1 * kRowBytes;
      constexpr int kBatch = 3;
      u32x4_t a[2][kBatch][2];
      auto read_a = [&](int s0, u32x4_t (&dst)[kBatch][2]) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int s = s0 + k;
          dst[k][0] = *reinterpret_cast<const u32x4_t*>(ap0 + aoff[0][s & 1] + 128 * (s >> 1));
          dst[k][1] = *reinterpret_cast<const u32x4_t*>(ap1 + aoff[1][s & 1] + 128 * (s >> 1));
        }
      };
      read_a(0, a[0]);
#pragma unroll
      for (int s0 = 0; s0 < kKSteps; s0 += kBatch) {
        const int cur = (s0 / kBatch) & 1;
        if (s0 + kBatch < kKSteps) read_a(s0 + kBatch, a[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const bf16x8_t qk = as_bf16x8(qreg[s0 + k]);
          const int par = (s0 + k) & 1;
          st[0][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[cur][k][0]), qk, st[0][par], 0, 0, 0);
          st[1][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[cur][k][1]), qk, st[1][par], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // score of row 32 th + 16 h + 4 grp + i of the tile for head col16
      float sc[8];
      float tmax = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = it * kTile + th * kHalf + 16 * h + 4 * grp + i;
          const float v = rows[tok] != kNoRow ? (st[h][0][i] + st[h][1][i]) * scale_log2 : kNegInf;
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
        // a few accumulators at a time (they live in AGPRs; the barriers keep the
        // scheduler from moving them all to VGPRs at once)
#pragma unroll
        for (int j = 0; j < kDimBlocks; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[j][i] *= a4[i];
          if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
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
      // O += P V, 32 blocks of 16 dims; the B operands (two transposing reads
      // each) in batches of 4 blocks, the next batch read before this one's MFMAs
      // piece 2 jb + vsub of a row sits at 128 (jb / 4) + voff[r][jb % 4]
      const uint8_t* vp0 = T + vrow0 * kRowBytes;
      const uint8_t* vp1 = T + vrow1 * kRowBytes;
      constexpr int kVB = 4;
      i16x4_t vb[2][kVB][2];
      auto read_v = [&](int j0, i16x4_t (&dst)[kVB][2]) {
#pragma unroll
        for (int k = 0; k < kVB; ++k) {
          const int jb = j0 + k;
          dst[k][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vp0 + voff[0][jb & 3] + 128 * (jb >> 2)));
          dst[k][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vp1 + voff[1][jb & 3] + 128 * (jb >> 2)));
        }
      };
      read_v(0, vb[0]);
#pragma unroll
      for (int j0 = 0; j0 < kDimBlocks; j0 += kVB) {
        const int cur = (j0 / kVB) & 1;
        if (j0 + kVB < kDimBlocks) read_v(j0 + kVB, vb[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kVB; ++k) {
          const bf16x8_t v = join_bf16x4(vb[cur][k][0], vb[cur][k][1]);
          oacc[j0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, v, oacc[j0 + k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kVB; ++k) {
          const bf16x8_t v = join_bf16x4(vb[cur][k][0], vb[cur][k][1]);
          oacc[j0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, oacc[j0 + k], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
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
  // wave through LDS (buffer hb of the ring, free once every wave is past the
  // last tile).
  constexpr int kXfer = kDimBlocks * 64 * 4 + 64 * 8;  // floats per head block
  static_assert(kXfer * 4 <= kTileBytes, "hand-over fits one tile buffer");
  float* xf = reinterpret_cast<float*>(hb ? buf1 : buf0);
  __syncthreads();
  if (th == 1) {
#pragma unroll
    for (int j = 0; j < kDimBlocks; ++j)
      *reinterpret_cast<f32x4_t*>(xf + (j * 64 + lane) * 4) = oacc[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[kDimBlocks * 256 + lane * 8 + i] = mh[i];
      xf[kDimBlocks * 256 + lane * 8 + 4 + i] = lh[i];
    }
  }
  __syncthreads();
  if (th == 1 || !active) return;
  float wa[4], wb[4], inv[4], lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mb = xf[kDimBlocks * 256 + lane * 8 + i];
    const float lb = xf[kDimBlocks * 256 + lane * 8 + 4 + i];
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
    float* dst = ws_o + unit * kDv + col16;
#pragma unroll
    for (int j = 0; j < kDimBlocks; ++j)
      dst[j * 16] = (oacc[j][i] * wa[i] + xf[(j * 64 + lane) * 4 + i] * wb[i]) * inv[i];
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

hipError_t launch_sparse(const void* q, const void* kv, const int32_t* indices, int B, int s_q,
                         int Hq, int s_kv, int d_qk, int d_v, int topk, float sm_scale,
                         float* out, float* lse, void* ws, int32_t* err_flag,
                         hipStream_t stream) {
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
                       indices, B, s_q, Hq, s_kv, topk, sm_scale * kLog2e, n_hg, n_splits,
                       per_hg, ws_o, ws_lse, err_flag);
  }
  hipLaunchKernelGGL(sparse_merge_kernel, dim3(B * Hq), dim3(256), 0, stream, ws_o, ws_lse,
                     n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace dakv
