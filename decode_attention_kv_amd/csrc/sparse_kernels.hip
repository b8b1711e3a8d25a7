// Top-k sparse MLA-style decode on the matrix cores (FlashMLA on Huawei Ascend,
// "Mathematical formulation" and "Course of computation"): all query heads of a
// sequence share the gathered latent rows G = kv[b][indices[b]] (d_qk = 576), the
// value is G[:, :512], and the softmax runs online over blocks of the index list
// with a running max that is only moved when it grows by more than a threshold
// ("skip scale").
//
// Work split: one workgroup (8 waves) per (sequence, 32 query heads, 512
// indices); the head groups of one (sequence, index split) sit a multiple of 8
// workgroups apart, so they run on one XCD and share its L2.  The 32 heads are
// two blocks of 16 (hb = wave / 4); within a head block, wave rb = wave % 4
// scores rows 16 rb .. 16 rb + 15 of every 64-row tile and accumulates output
// dims 128 rb .. 128 rb + 127 over all 64 rows, so the accumulators of a wave
// are 16 heads x 128 dims and two waves fit each SIMD.
//   * Rows are gathered by direct-to-LDS buffer loads (16 bytes per lane, no
//     registers) into two tile buffers: tile it + 1 is in flight while tile it is
//     computed, its loads issued in three parts over tile it.  A tile is 64 unpadded
//     1152-byte rows; the 16-byte pieces of row r are stored in a permuted order
//     (the piece's low 3 bits XOR (r / 2) % 8). On this chip's LDS, which serves 32
//     lanes of a 16-byte read per pass from 512-byte bank rows (measured), that puts
//     the 32 pieces each pass reads (16 rows x an aligned pair of pieces, for both
//     read patterns below) in distinct banks.
//   * S^T[token, head] = G Q^T with v_mfma_f32_16x16x32_bf16: A = the wave's 16
//     rows x 32 dims from LDS (read a batch of k-steps ahead), B = Q^T of the
//     wave's 16 heads, held in registers for the whole split (18 k-steps x 16
//     bytes per lane); three accumulation chains.
//   * Each wave exponentiates its own 16 rows against the running max the four
//     waves of a head block share, and publishes P (as bf16 hi + lo parts) with
//     its rows' max through LDS (one barrier per tile).  Only when a tile raises
//     a max by more than the skip-scale threshold (the first tile always does)
//     does the whole workgroup move the max, rescale and publish again.
//   * The C layout of S^T (lane: head lane % 16, tokens 4 (lane / 16) + i of a
//     row block) is the A layout of P for O = P V when the 8 tokens of a lane
//     group in k-step kk are tokens {4g..4g+3} of row blocks 2 kk and 2 kk + 1,
//     so each lane reads its P operands as published.  P enters the matrix core
//     as bf16 hi + lo parts (two MFMAs per block).
//   * The B operand of P V (8 rows of one dim per lane) comes straight from LDS
//     with two transposing reads ds_read_b64_tr_b16: lane j of a 16-lane group
//     points at row 4 (group) + j / 4 (+16), dims 4 (j % 4) .. +3 of a 16-dim
//     block, and lane i receives dim i of that block for the 4 rows.
// At the end each wave writes its dims of o / l (and one wave the log2-sum-exp);
// a merge kernel combines the splits.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;                     // 1152
constexpr int kPieces = kRowBytes / 16;                 // 72 pieces of 16 bytes
constexpr int kTile = 64;                               // gathered rows per tile
constexpr int kTileBytes = kTile * kRowBytes;           // 73728
constexpr int kSplit = 512;                             // indices per workgroup
constexpr int kSpWaves = 8;
constexpr int kSpThreads = kSpWaves * 64;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 32;
constexpr int kRowBlock = 16;                           // tile rows one wave scores
constexpr int kRowBlocks = kTile / kRowBlock;           // 4 waves per head block
constexpr int kDmaPerWave = kTileBytes / 1024 / kSpWaves;  // 9 wave loads of 1 KiB per tile
// The next tile's gather is spread over the tile (a wave's loads [0, kGatherTop) at its
// top, [kGatherTop, kGatherMid) once the scores are in, the rest after the P
// exchange), so that the rows landing in LDS compete less with the scores' operand
// reads.  Measured per call (bf16 rows): all at the top 36.5 us; 3 / 6 35.0; 2 / 4 / 3
// 34.2 (1 / 3 / 5 and 1 / 4 / 4 34.7; 2 / 3 / 4 34.8).
constexpr int kGatherTop = 2;
constexpr int kGatherMid = 6;
constexpr int kKSteps = kDqk / 32;                      // 18
constexpr int kDimsPerWave = kDv / kRowBlocks;          // 128 output dims per wave
constexpr int kWaveDimBlocks = kDimsPerWave / 16;       // 8 blocks of 16 dims
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = (0 & 15) | (7 << 4) | (15 << 8);    // vmcnt(0) only
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0) only
// The page's rescale threshold is 6 in natural-log units; scores here are in log2.
constexpr float kRescale = 6.0f * kLog2e;
constexpr uint32_t kNoRow = 0x80000000u;  // a buffer offset past any sequence: loads 0
static_assert(kTileBytes % (1024 * kSpWaves) == 0, "whole 1 KiB wave loads per wave");
static_assert(2 * kHeadsPerWave == kHeadsPerWG && kRowBlocks * 2 == kSpWaves,
              "two head blocks of four waves");
static_assert(kPieces % 8 == 0, "pieces permute within groups of 8");
static_assert(kSplit % kTile == 0, "whole tiles per split");

// Position of piece p of row r inside the row (an involution: it also maps a
// position back to its piece).
__device__ __forceinline__ int piece_slot(int p, int r) {
  return (p & ~7) | ((p & 7) ^ ((r >> 1) & 7));
}

// Barrier for values exchanged through LDS by ordinary stores: waits for this
// wave's LDS accesses but not for its buffer loads, so the next tile's gather
// stays in flight (an LDS release fence would also wait for those, since they
// write LDS).  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Max and sum over the 4 lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with the
// row-swap instructions, without an LDS round trip: after a swap of x with itself a
// lane holds {x[l], x[l ^ 16]} (v_permlane16_swap) or {x[l], x[l ^ 32]}
// (v_permlane32_swap), in an order that does not matter here (checked on the
// device).
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t join_bf16x4(const i16x4_t& lo, const i16x4_t& hi) {
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Latent cache formats: bf16 rows, or codes with one fp32 scale per row -- E4M3
// (one byte a value) or E2M1 (two values a byte, element 2i in the low four bits).
// For codes, the tile buffers keep the bf16 layout of the bf16 cache: each thread
// loads its code pieces of the next tile into registers while the current tile is
// computed, then stores them as code value times row scale (exact in bf16, the
// scale being a power of two) at the permuted piece positions.
enum LatentFormat : int { kLatentBf16 = 0, kLatentFp8 = 1, kLatentFp4 = 2 };

template <int kFmt>
__global__ void __launch_bounds__(kSpThreads)
sparse_split_kernel(const uint16_t* __restrict__ q, const void* __restrict__ kv,
                    const float* __restrict__ kv_scale, const int32_t* __restrict__ indices,
                    int B, int s_q, int Hq, int s_kv, int topk, float scale_log2, int n_hg,
                    int n_splits, int per_hg, float* __restrict__ ws_o,
                    float* __restrict__ ws_lse, int32_t* err_flag) {
  constexpr bool kCodes = kFmt != kLatentBf16;
  constexpr int kSrcRowBytes = kFmt == kLatentBf16 ? kRowBytes     // a latent row in the cache
                               : kFmt == kLatentFp8 ? kDqk : kDqk / 2;
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[kTileBytes];
  __shared__ uint32_t rows[kSplit];  // byte offset of each index's row in kv[b], or kNoRow
  __shared__ float row_scale[kCodes ? kSplit : 1];       // codes: each index's row scale
  // P of each row block (bf16 hi parts in .xy, lo parts in .zw; lane layout of the
  // block's scores), each row block's score max per head, the waves' rescale flags
  // and, at the end, each row block's sum of exponentials per head
  __shared__ u32x4_t sm_p[2][kRowBlocks][64];
  __shared__ float sm_mx[2][kRowBlocks][16];
  __shared__ int sm_flag[kSpWaves];
  __shared__ float sm_l[2][kRowBlocks][16];
  const int hg = blockIdx.x / per_hg;
  const int u = blockIdx.x - hg * per_hg;
  if (u >= B * n_splits) return;
  const int b = u / n_splits;
  const int split = u - b * n_splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave >> 2;    // head block of the group
  const int rb = wave & 3;     // row block of every tile (scores), dim quarter (P V)
  const int grp = lane >> 4;   // lane group 0..3
  const int col16 = lane & 15;
  const int head0 = hg * kHeadsPerWG + hb * kHeadsPerWave;
  const int t0 = split * kSplit;
  const int ntok = min(kSplit, topk - t0);
  // Q of the workgroup's 32 heads (36 KiB, contiguous in q) is gathered once into
  // buf1, which is free until tile 1, in the tile layout (head r of the group as
  // row r, its pieces permuted by piece_slot); every wave then reads its Q^T
  // operands from there.  (Loading them straight from memory had each Q value
  // fetched by the 4 waves of a head block and the 4 index splits of a sequence.)
  // Positions past the 32 heads, and heads past Hq, are filled with zeros.  The
  // offsets are computed first, this thread's index load is issued next, and the
  // gather after it, so that waiting for the index does not wait for the gather.
  constexpr int kQPieces = kHeadsPerWG * kPieces;                         // 2304
  constexpr int kQLoads = (kQPieces + kSpThreads - 1) / kSpThreads;       // 5 per wave
  static_assert(kQLoads * kSpThreads * 16 <= kTileBytes, "Q fits one tile buffer");
  static_assert(kSplit == kSpThreads, "one index per thread");
  uint32_t qoff[kQLoads];
#pragma unroll
  for (int k = 0; k < kQLoads; ++k) {
    const uint32_t c = (uint32_t)((k * kSpWaves + wave) * 64 + lane);
    const uint32_t r = c / kPieces;
    const int p = piece_slot((int)(c - r * kPieces), (int)r);
    qoff[k] = r < kHeadsPerWG ? (hg * kHeadsPerWG + r) * kRowBytes + (uint32_t)p * 16 : kNoRow;
    asm volatile("" : "+v"(qoff[k]));  // computed here, before the index load
  }
  const int my_idx = tid < ntok ? indices[(size_t)b * topk + t0 + tid] : -1;
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + (size_t)b * Hq * kDqk, (short)0, Hq * kRowBytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < kQLoads; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qr, (lds_void*)(buf1 + (k * kSpWaves + wave) * 1024), 16, (int)qoff[k], 0, 0, 0);
  }
  {
    uint32_t r = kNoRow;
    float sc = 0.f;
    if (tid < ntok) {
      if (my_idx >= 0 && my_idx < s_kv) {
        r = (uint32_t)my_idx * kSrcRowBytes;
        if constexpr (kCodes) sc = kv_scale[(size_t)(b / s_q) * s_kv + my_idx];
      } else {
        raise_flag(err_flag, 4);
      }
    }
    rows[tid] = r;
    if constexpr (kCodes) row_scale[tid] = sc;
  }
  lds_barrier();
  // the sequence's latent rows as a buffer (the q-tokens of one sequence, b / s_q,
  // share them): an absent row reads as zeros
  const __amdgpu_buffer_rsrc_t kvr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(kv)) +
          (size_t)(b / s_q) * s_kv * kSrcRowBytes,
      (short)0, (int)(s_kv * kSrcRowBytes), 0x00020000);
  const int ntiles = (ntok + kTile - 1) / kTile;

  // Tile ti into a buffer: wave load I (this wave's I = 9 wave + k) fills bytes
  // [1024 I, 1024 I + 1024) of the tile, lane L the 16 bytes at 1024 I + 16 L,
  // i.e. position c = 64 I + L = 72 r + s of row r, which holds piece
  // piece_slot(s, r).  Rows past the split's end load kNoRow offsets (zeros).
  auto fetch_tile = [&](int ti, uint8_t* dst, int k0, int k1) {  // this wave's loads [k0, k1)
    uint32_t off[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      if (k < k0 || k >= k1) continue;
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
      if (k < k0 || k >= k1) continue;
      const int I = wave * kDmaPerWave + k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kvr, (lds_void*)(dst + I * 1024), 16, (int)off[k],
                                               0, 0, 0);
    }
  };
  // Codes: thread t holds the code pieces c = t + 512 k of a tile (row c / P, P
  // pieces a row: 36 of 16 bytes = 16 E4M3 values, or 36 of 8 bytes = 16 E2M1
  // values), loaded by load_codes and stored converted by store_codes as the two
  // bf16 pieces of those values.  The LDS stores of one instruction then sit 32
  // bytes apart across lanes (two lanes a bank group); E2M1 pieces of 16 bytes
  // (four bf16 pieces each, 64 bytes apart: four lanes a bank group) measured
  // 38.1 against 36.0 us per call, 4-byte E2M1 and 8-byte E4M3 pieces (one bf16
  // piece a lane, twice the loads) 36.5 and 38.6 us.
  constexpr int kCodeBytes = kFmt == kLatentFp4 ? 8 : 16;
  constexpr int kCodeWords = kCodeBytes / 4;
  constexpr int kPiecesPerCode = kFmt == kLatentFp4 ? kCodeBytes / 4 : kCodeBytes / 8;
  constexpr int kCodePiecesRow = kSrcRowBytes / kCodeBytes;
  constexpr int kCodePieces = kTile * kCodePiecesRow;
  constexpr int kCodesPerThread = (kCodePieces + kSpThreads - 1) / kSpThreads;
  static_assert(kCodePiecesRow * kCodeBytes == kSrcRowBytes, "whole code pieces a row");
  uint32_t creg[kCodes ? kCodesPerThread : 1][kCodeWords];
  auto load_codes = [&](int ti) {
#pragma unroll
    for (int k = 0; k < kCodesPerThread; ++k) {
      const int c = tid + kSpThreads * k;
      const int r = c / kCodePiecesRow;
      const uint32_t o = c < kCodePieces ? rows[ti * kTile + r] : kNoRow;
      const uint32_t off = o == kNoRow ? kNoRow : o + (uint32_t)(c - r * kCodePiecesRow) * kCodeBytes;
      if constexpr (kCodeBytes == 16) {
        const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(kvr, (int)off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) creg[k][i] = w[i];
      } else {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(kvr, (int)off, 0, 0);
        creg[k][0] = w[0];
        creg[k][1] = w[1];
      }
    }
  };
  auto store_codes = [&](int ti, uint8_t* dst) {
#pragma unroll
    for (int k = 0; k < kCodesPerThread; ++k) {
      const int c = tid + kSpThreads * k;
      if (c < kCodePieces) {
        const int r = c / kCodePiecesRow;
        const int pp = c - r * kCodePiecesRow;
        const float sc = row_scale[ti * kTile + r];
        uint8_t* row = dst + r * kRowBytes;
#pragma unroll
        for (int qq = 0; qq < kPiecesPerCode; ++qq) {
          // E4M3: words 2 qq, 2 qq + 1 hold values 8 qq .. 8 qq + 7 (bytes in memory
          // order); E2M1: word qq holds them, byte j values 8 qq + 2 j (low four
          // bits) and 8 qq + 2 j + 1
          u32x4_t h;
          if constexpr (kFmt == kLatentFp8) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              h[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(creg[k][2 * qq + w], sc, false));
              h[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(creg[k][2 * qq + w], sc, true));
            }
          } else {
            h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(creg[k][qq], sc, 0));
            h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(creg[k][qq], sc, 1));
            h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(creg[k][qq], sc, 2));
            h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(creg[k][qq], sc, 3));
          }
          *reinterpret_cast<u32x4_t*>(row + piece_slot(kPiecesPerCode * pp + qq, r) * 16) = h;
        }
      }
    }
  };
  if constexpr (kCodes) load_codes(0);
  else fetch_tile(0, buf0, 0, kDmaPerWave);
  // Q^T of the wave's heads as B operands, read from buf1 once its gather is
  // complete: lane -> head head0 + col16 (row hb * 16 + col16 of buf1), dims
  // 32 s + 8 grp .. +8.  All reads are done before tile 1's gather refills buf1.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4_t qreg[kKSteps];
  {
    const int qrow = hb * kHeadsPerWave + col16;
    const uint8_t* qp = buf1 + qrow * kRowBytes;
    const int q0 = piece_slot(grp, qrow) * 16, q1 = piece_slot(4 + grp, qrow) * 16;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      qreg[s] = *reinterpret_cast<const u32x4_t*>(qp + ((s & 1) ? q1 : q0) + 128 * (s >> 1));
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  if constexpr (kCodes) store_codes(0, buf0);

  // O of the wave's 16 heads and its 128 output dims (C layout: lane -> dim
  // 16 j + col16 of dim block 8 rb + j, heads 4 grp + i)
  f32x4_t oacc[kWaveDimBlocks];
#pragma unroll
  for (int j = 0; j < kWaveDimBlocks; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // running max used for the exponentials (head head0 + col16; the same in the
  // four waves of a head block) and this lane's share of the sum of exponentials
  float m_ref = kNegInf;
  float lsum = 0.f;

  // A operand of k-step s: row 16 rb + col16, piece 4 s + grp, which sits at
  // byte 128 (s / 2) + aoff[s % 2] of the row (the permutation only moves a piece
  // inside its group of 8).
  const int arow = rb * kRowBlock + col16;
  int aoff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) aoff[par] = piece_slot(4 * par + grp, arow) * 16;
  // Transposing reads for k-step kk of P V, half r: rows 32 kk + 16 r + 4 grp +
  // col16 / 4, dims 16 jb + 4 (col16 % 4) .. +3 of dim block jb: piece 2 jb +
  // (col16 % 4) / 2, byte 8 (col16 & 1) of it.
  const int vsub = (col16 & 3) >> 1;
  const int vhalf = (col16 & 1) * 8;
  int vbase[2][2];
  int voff[2][2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int vrow = 32 * kk + 16 * r + 4 * grp + (col16 >> 2);
      vbase[kk][r] = vrow * kRowBytes + 256 * rb;  // dim block 8 rb starts piece group 2 rb
#pragma unroll
      for (int j = 0; j < 4; ++j) voff[kk][r][j] = piece_slot(2 * j + vsub, vrow) * 16 + vhalf;
    }
  }

  // One tile: T holds it, N receives the next.  (Called with the two buffers
  // named at compile time, so the compiler sees that reads of T do not touch the
  // gather in flight into N and does not wait for it.)
  auto tile = [&](int it, const uint8_t* T, uint8_t* N) {
    // this wave's loads of tile it are complete (none later is in flight yet);
    // the barrier makes every wave's part visible and ends every wave's reads of
    // tile it - 1, whose buffer the next fetch refills
    // (codes: this wave's converted stores of tile it are complete.)
    if constexpr (kCodes) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 1 < ntiles) {
      if constexpr (kCodes) load_codes(it + 1);
      else fetch_tile(it + 1, N, 0, kGatherTop);
    }

    // S^T = G Q^T for the wave's 16 rows over 18 k-steps in three chains; A
    // operands read from LDS a batch of 3 k-steps ahead
    f32x4_t st[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) st[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* ap = T + arow * kRowBytes;
      constexpr int kBatch = 3;
      u32x4_t a[2][kBatch];
      auto read_a = [&](int s0, u32x4_t (&dst)[kBatch]) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int s = s0 + k;
          dst[k] = *reinterpret_cast<const u32x4_t*>(ap + aoff[s & 1] + 128 * (s >> 1));
        }
      };
      read_a(0, a[0]);
#pragma unroll
      for (int s0 = 0; s0 < kKSteps; s0 += kBatch) {
        const int cur = (s0 / kBatch) & 1;
        if (s0 + kBatch < kKSteps) read_a(s0 + kBatch, a[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
          st[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[cur][k]),
                                                          as_bf16x8(qreg[s0 + k]), st[k], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!kCodes) {
      if (it + 1 < ntiles) fetch_tile(it + 1, N, kGatherTop, kGatherMid);
    }
    // scores of this wave's tile rows 16 rb + 4 grp + i for head col16 (-inf for
    // rows past the index list), and their max per head
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = it * kTile + rb * kRowBlock + 4 * grp + i;
      sc[i] = rows[tok] != kNoRow ? (st[0][i] + st[1][i] + st[2][i]) * scale_log2 : kNegInf;
    }
    const float bmax = group4_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    // skip-scale: the exponentials of this wave's rows are taken against the running
    // max m_ref as it stands; a tile that raises it by more than the threshold in
    // any row block (the first tile always does) is redone below for the whole
    // workgroup, so that every wave passes the same barriers
    auto publish = [&](float mu) {
      u32x4_t pk;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = exp2_fast(sc[i] - mu), p1 = exp2_fast(sc[i + 1] - mu);
        ps += p0 + p1;
        const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
        const bf16x2_t hh = {h0, h1};
        const bf16x2_t ll = {(__bf16)(p0 - (float)h0), (__bf16)(p1 - (float)h1)};
        pk[i >> 1] = __builtin_bit_cast(uint32_t, hh);
        pk[2 + (i >> 1)] = __builtin_bit_cast(uint32_t, ll);
      }
      sm_p[hb][rb][lane] = pk;
      return ps;
    };
    const bool raise = __any(bmax > m_ref + kRescale);
    // V operands of the first k-step of P V, read while the exponentials are taken
    // and the waves meet (they do not depend on P): the transposing reads bound the
    // P V phase, and the LDS is otherwise idle in this one (bf16 rows: 37.3 against
    // 38.0 us per call, 255 VGPRs; the code formats, which hold the next tile's codes
    // in registers here, would spill)
    i16x4_t vb0[kWaveDimBlocks][2];
    if constexpr (!kCodes) {
#pragma unroll
      for (int j = 0; j < kWaveDimBlocks; ++j) {
        vb0[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + vbase[0][0] + voff[0][0][j & 3] + 128 * (j >> 2)));
        vb0[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + vbase[0][1] + voff[0][1][j & 3] + 128 * (j >> 2)));
      }
    }
    float psum = publish(m_ref == kNegInf ? 0.f : m_ref);
    if (grp == 0) sm_mx[hb][rb][col16] = bmax;
    if (lane == 0) sm_flag[wave] = raise;
    lds_barrier();
    bool redo = false;
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) redo |= sm_flag[w] != 0;
    if (redo) {  // rare: the running max moves (the same decision in every wave)
      float tmax = kNegInf;
#pragma unroll
      for (int b4 = 0; b4 < kRowBlocks; ++b4) tmax = fmaxf(tmax, sm_mx[hb][b4][col16]);
      const float mnew = fmaxf(m_ref, tmax);
      const float alpha = mnew == kNegInf ? 1.f : exp2_fast(m_ref - mnew);
      lsum *= alpha;
      m_ref = mnew;
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
      for (int j = 0; j < kWaveDimBlocks; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[j][i] *= a4[i];
      }
      // (no wave reads P before the barrier below, so it can be rewritten now)
      psum = publish(m_ref == kNegInf ? 0.f : m_ref);
      lds_barrier();
    }
    lsum += psum;
    if constexpr (!kCodes) {
      if (it + 1 < ntiles) fetch_tile(it + 1, N, kGatherMid, kDmaPerWave);
    }

    // O += P V over the tile's 64 rows for dim blocks 8 rb .. 8 rb + 7.  k-step
    // kk: lane group g holds tokens {4g..4g+3} of row blocks 2 kk and 2 kk + 1
    // (the published P of those blocks, in their scores' lane layout), and the
    // transposing reads return V rows in the same order.  P enters as two bf16
    // parts (p = hi + lo to about 16 significant bits): rounding P to one bf16
    // alone can put the output off by more than 2e-3 when a few rows dominate the
    // softmax.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4_t q0 = sm_p[hb][2 * kk][lane], q1 = sm_p[hb][2 * kk + 1][lane];
      const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, u32x4_t{q0[0], q0[1], q1[0], q1[1]});
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, u32x4_t{q0[2], q0[3], q1[2], q1[3]});
      const uint8_t* vp0 = T + vbase[kk][0];
      const uint8_t* vp1 = T + vbase[kk][1];
      i16x4_t vb[kWaveDimBlocks][2];
#pragma unroll
      for (int j = 0; j < kWaveDimBlocks; ++j) {
        if (!kCodes && kk == 0) {
          vb[j][0] = vb0[j][0];
          vb[j][1] = vb0[j][1];
          continue;
        }
        vb[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vp0 + voff[kk][0][j & 3] + 128 * (j >> 2)));
        vb[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vp1 + voff[kk][1][j & 3] + 128 * (j >> 2)));
      }
#pragma unroll
      for (int j = 0; j < kWaveDimBlocks; ++j) {
        const bf16x8_t v = join_bf16x4(vb[j][0], vb[j][1]);
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, v, oacc[j], 0, 0, 0);
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, oacc[j], 0, 0, 0);
      }
    }
    if constexpr (kCodes) {
      if (it + 1 < ntiles) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        store_codes(it + 1, N);
      }
    }
  };
  for (int it = 0; it < ntiles; it += 2) {
    tile(it, buf0, buf1);
    if (it + 1 < ntiles) tile(it + 1, buf1, buf0);
  }

  // Epilogue.  The sum of exponentials per head: each wave summed its own row
  // block's, against the running max that the four waves of a head block share.
  lsum = group4_sum(lsum);
  if (grp == 0) sm_l[hb][rb][col16] = lsum;
  lds_barrier();
  lsum = sm_l[hb][0][col16] + sm_l[hb][1][col16] + sm_l[hb][2][col16] + sm_l[hb][3][col16];
  float inv[4], lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = __shfl(lsum, 4 * grp + i);
    const float M = __shfl(m_ref, 4 * grp + i);
    if (M == kNegInf) {
      inv[i] = 0.f;
      lse2[i] = kNegInf;
    } else {
      inv[i] = 1.f / l;
      lse2[i] = M + __log2f(l);
    }
  }
  if (head0 >= Hq) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = head0 + 4 * grp + i;
    const size_t unit = ((size_t)b * Hq + head) * n_splits + split;
    float* dst = ws_o + unit * kDv + rb * kDimsPerWave + col16;
#pragma unroll
    for (int j = 0; j < kWaveDimBlocks; ++j) dst[j * 16] = oacc[j][i] * inv[i];
    if (rb == 0 && col16 == 0) ws_lse[unit] = lse2[i];
  }
}

// Combine the splits of one (sequence, head): weights 2^(lse_j - max).  Splits
// are taken 8 at a time; each thread issues its log-sum-exp and partial loads of
// a batch together, so a head of up to 8 splits takes one memory round trip
// (running max and sums rescaled from batch to batch).
constexpr int kMergeBatch = 8;
static_assert(kDv == 2 * 256, "two columns per thread");

__global__ void __launch_bounds__(256)
sparse_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    int n_splits, float* __restrict__ out, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* lp = ws_lse + (size_t)bh * n_splits;
  const float* op = ws_o + (size_t)bh * n_splits * kDv;
  const int d0 = threadIdx.x * 2;  // two adjacent columns per thread
  float M = kNegInf, num0 = 0.f, num1 = 0.f, den = 0.f;
  for (int j0 = 0; j0 < n_splits; j0 += kMergeBatch) {
    float x[kMergeBatch];
    float2 v[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const bool in = j0 + k < n_splits;
      x[k] = in ? lp[j0 + k] : kNegInf;
      v[k] = in ? *reinterpret_cast<const float2*>(op + (size_t)(j0 + k) * kDv + d0)
                : make_float2(0.f, 0.f);
    }
    float m = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) m = fmaxf(m, x[k]);
    if (m == kNegInf) continue;  // nothing attended yet
    const float r = exp2_fast(M - m);  // 0 while M is -inf
    num0 *= r;
    num1 *= r;
    den *= r;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wk = exp2_fast(x[k] - m);
      num0 += wk * v[k].x;
      num1 += wk * v[k].y;
      den += wk;
    }
    M = m;
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

hipError_t launch_sparse(const void* q, const void* kv, const float* kv_scale, int format,
                         const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                         int d_v, int topk, float sm_scale, float* out, float* lse, void* ws,
                         int32_t* err_flag, hipStream_t stream) {
  (void)d_qk;
  (void)d_v;
  const int n_splits = sparse_splits(topk);
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o + (size_t)B * Hq * n_splits * kDv;
  if (n_splits > 0) {
    const int n_hg = (Hq + kHeadsPerWG - 1) / kHeadsPerWG;
    const int per_hg = (B * n_splits + 7) / 8 * 8;
    const dim3 grid(n_hg * per_hg), block(kSpThreads);
    const float sl = sm_scale * kLog2e;
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    if (format == kLatentFp8)
      hipLaunchKernelGGL(sparse_split_kernel<kLatentFp8>, grid, block, 0, stream, q16, kv,
                         kv_scale, indices, B, s_q, Hq, s_kv, topk, sl, n_hg, n_splits, per_hg,
                         ws_o, ws_lse, err_flag);
    else if (format == kLatentFp4)
      hipLaunchKernelGGL(sparse_split_kernel<kLatentFp4>, grid, block, 0, stream, q16, kv,
                         kv_scale, indices, B, s_q, Hq, s_kv, topk, sl, n_hg, n_splits, per_hg,
                         ws_o, ws_lse, err_flag);
    else
      hipLaunchKernelGGL(sparse_split_kernel<kLatentBf16>, grid, block, 0, stream, q16, kv,
                         nullptr, indices, B, s_q, Hq, s_kv, topk, sl, n_hg, n_splits, per_hg,
                         ws_o, ws_lse, err_flag);
  }
  hipLaunchKernelGGL(sparse_merge_kernel, dim3(B * Hq), dim3(256), 0, stream, ws_o, ws_lse,
                     n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace dakv
