// The FP8 KV cache: E4M3 codes (one byte per element) with a power-of-two fp32
// scale per cached row, for K and for V, in the static layout ([B, H, cap, D]
// codes, [B, H, cap] scales) and in the paged pool ([num_blocks, block_size, Hkv,
// D] codes, [num_blocks, block_size, Hkv] scales).  The appends quantise a new
// token's rows; the split passes read codes and scales and feed the same split-K
// machinery (workspace, merge) as the bf16 caches.
#include "split_common.hpp"

namespace dakv {

// ---------------------------------------------------------------------------
// kv_append_fp8: the new token's K and V rows are quantised to E4M3 codes with a
// power-of-two scale per row and stored at row write_pos[b].  One wave per
// (sequence, head, K or V): the row's largest magnitude comes from a wave
// reduction; the scale is 2^e with e the smallest integer for which
// max|x| <= 448 * 2^e (from the exponent and fraction of max|x|, exactly); each
// value x * 2^-e (exact) is rounded to the nearest E4M3 value, ties to the even
// code, zero results as the +0 code.
// ---------------------------------------------------------------------------
// One wave quantises one row of D <= 64 kPer bf16 values: codes to dst, scale to
// *dst_scale.
template <int kPer>
__device__ __forceinline__ void quantise_row_wave(const uint16_t* __restrict__ src, int D,
                                                  uint8_t* __restrict__ dst,
                                                  float* __restrict__ dst_scale, int lane) {
  float x[kPer];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {         // at most kPer values per lane
    const int d = lane + 64 * i;
    x[i] = d < D ? __uint_as_float((uint32_t)src[d] << 16) : 0.f;
    amax = fmaxf(amax, fabsf(x[i]));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int e = e4m3_exponent_for(amax);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int d = lane + 64 * i;
    if (d < D) dst[d] = (uint8_t)e4m3_code(ldexpf(x[i], -e));
  }
  if (lane == 0) *dst_scale = ldexpf(1.f, e);
}

__global__ void __launch_bounds__(256)
kv_append_fp8_kernel(uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes,
                     float* __restrict__ k_scale, float* __restrict__ v_scale,
                     const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                     const int32_t* __restrict__ write_pos, int32_t* __restrict__ mask, int H,
                     int cap, int D, int32_t* err_flag) {
  const int b = blockIdx.y;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);  // (head, K or V)
  const int lane = threadIdx.x & 63;
  if (unit >= 2 * H) return;
  const int h = unit >> 1;
  const bool is_v = unit & 1;
  const int pos = write_pos[b];
  if (pos < 0 || pos >= cap) {
    if (unit == 0 && lane == 0) raise_flag(err_flag, 2);
    return;
  }
  const uint16_t* src = (is_v ? v_new : k_new) + ((size_t)b * H + h) * D;
  const size_t row = ((size_t)b * H + h) * cap + pos;
  quantise_row_wave<4>(src, D, (is_v ? v_codes : k_codes) + row * D,
                    (is_v ? v_scale : k_scale) + row, lane);
  if (mask && unit == 0 && lane == 0) mask[(size_t)b * cap + pos] = 1;
}

hipError_t launch_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                const void* k_new, const void* v_new, const int32_t* write_pos,
                                int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                                hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((2 * H + 3) / 4, B), dim3(256), 0, stream,
                     static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes), k_scale,
                     v_scale, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), write_pos, mask, H, cap, D, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// latent_append_fp8: each sequence's new latent row (bf16, d <= 576 values) is
// quantised as kv_append_fp8 quantises a K or V row and stored at row
// write_pos[b] of that sequence's latent cache (codes [B, s_kv, d], scales
// [B, s_kv]).  One wave per sequence.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
latent_append_fp8_kernel(uint8_t* __restrict__ codes, float* __restrict__ scale,
                         const uint16_t* __restrict__ new_rows,
                         const int32_t* __restrict__ write_pos, int B, int s_kv, int d,
                         int32_t* err_flag) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  const int pos = write_pos[b];
  if (pos < 0 || pos >= s_kv) {
    if (lane == 0) raise_flag(err_flag, 2);
    return;
  }
  const size_t row = (size_t)b * s_kv + pos;
  quantise_row_wave<9>(new_rows + (size_t)b * d, d, codes + row * d, scale + row, lane);
}

hipError_t launch_latent_append_fp8(void* codes, float* scale, const void* new_rows,
                                    const int32_t* write_pos, int B, int s_kv, int d,
                                    int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(latent_append_fp8_kernel, dim3((B + 3) / 4), dim3(256), 0, stream,
                     static_cast<uint8_t*>(codes), scale, static_cast<const uint16_t*>(new_rows),
                     write_pos, B, s_kv, d, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// kv_append_fp4: as kv_append_fp8 with E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3,
// 4, 6; scale 2^e with e the smallest integer for which max|x| <= 6 * 2^e), two
// codes per byte, element 2i in the low four bits.  One wave per (sequence, head,
// K or V); lane l quantises elements 2l and 2l + 1 (and 2l + 128, 2l + 129).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int e2m1_exponent_for(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);        // amax = f 2^E, f in [0.5, 1); 6 = 0.75 2^3
  return f <= 0.75f ? E - 3 : E - 2;
}

// |y| <= 6: the nearest E2M1 magnitude, counted by the midpoints it passes; a
// midpoint between codes goes to the even one (<= below an even code, < above).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t code = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) +
                        (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                        (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return (code != 0 && y < 0.f) ? (code | 8u) : code;
}

// One wave quantises one row of D <= 128 kPairs bf16 values to E2M1: lane l takes
// the value pairs (2p, 2p + 1) for p = l + 64 k and writes their byte p.
template <int kPairs>
__device__ __forceinline__ void quantise_row_wave_fp4(const uint16_t* __restrict__ src, int D,
                                                      uint8_t* __restrict__ dst,
                                                      float* __restrict__ dst_scale, int lane) {
  float x[2 * kPairs];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2 * kPairs; ++i) {
    const int v = 2 * (lane + 64 * (i >> 1)) + (i & 1);
    x[i] = v < D ? __uint_as_float((uint32_t)src[v] << 16) : 0.f;
    amax = fmaxf(amax, fabsf(x[i]));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int e = e2m1_exponent_for(amax);
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int p = lane + 64 * k;
    if (2 * p < D)
      dst[p] = (uint8_t)(e2m1_code(ldexpf(x[2 * k], -e)) |
                         (e2m1_code(ldexpf(x[2 * k + 1], -e)) << 4));
  }
  if (lane == 0) *dst_scale = ldexpf(1.f, e);
}

__global__ void __launch_bounds__(256)
kv_append_fp4_kernel(uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes,
                     float* __restrict__ k_scale, float* __restrict__ v_scale,
                     const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                     const int32_t* __restrict__ write_pos, int32_t* __restrict__ mask, int H,
                     int cap, int D, int32_t* err_flag) {
  const int b = blockIdx.y;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);  // (head, K or V)
  const int lane = threadIdx.x & 63;
  if (unit >= 2 * H) return;
  const int h = unit >> 1;
  const bool is_v = unit & 1;
  const int pos = write_pos[b];
  if (pos < 0 || pos >= cap) {
    if (unit == 0 && lane == 0) raise_flag(err_flag, 2);
    return;
  }
  const size_t row = ((size_t)b * H + h) * cap + pos;
  quantise_row_wave_fp4<2>((is_v ? v_new : k_new) + ((size_t)b * H + h) * D, D,
                           (is_v ? v_codes : k_codes) + row * (D / 2),
                           (is_v ? v_scale : k_scale) + row, lane);  // D <= 256
  if (mask && unit == 0 && lane == 0) mask[(size_t)b * cap + pos] = 1;
}

hipError_t launch_kv_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                const void* k_new, const void* v_new, const int32_t* write_pos,
                                int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                                hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_fp4_kernel, dim3((2 * H + 3) / 4, B), dim3(256), 0, stream,
                     static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes), k_scale,
                     v_scale, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), write_pos, mask, H, cap, D, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// latent_append_fp4: as latent_append_fp8 with E2M1 codes (the scale and rounding
// of kv_append_fp4), two codes per byte.  One wave per sequence; lane l quantises
// the value pairs (2p, 2p + 1) for p = l + 64 k.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
latent_append_fp4_kernel(uint8_t* __restrict__ codes, float* __restrict__ scale,
                         const uint16_t* __restrict__ new_rows,
                         const int32_t* __restrict__ write_pos, int B, int s_kv, int d,
                         int32_t* err_flag) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  const int pos = write_pos[b];
  if (pos < 0 || pos >= s_kv) {
    if (lane == 0) raise_flag(err_flag, 2);
    return;
  }
  const size_t row = (size_t)b * s_kv + pos;
  quantise_row_wave_fp4<5>(new_rows + (size_t)b * d, d, codes + row * (d / 2), scale + row,
                           lane);  // d <= 640
}

hipError_t launch_latent_append_fp4(void* codes, float* scale, const void* new_rows,
                                    const int32_t* write_pos, int B, int s_kv, int d,
                                    int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(latent_append_fp4_kernel, dim3((B + 3) / 4), dim3(256), 0, stream,
                     static_cast<uint8_t*>(codes), scale, static_cast<const uint16_t*>(new_rows),
                     write_pos, B, s_kv, d, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------- static layout, FP8
// Split pass of decode_attn_static_fp8: the cache holds E4M3 codes (one byte per
// element, [B, H, cap, D]) and one power-of-two fp32 scale per row for K and for V
// ([B, H, cap]).  A lane covers 8 elements of a row as in the bf16 kernel (D / 8
// lanes per row), now 8 bytes: K and V codes arrive by 8-byte buffer loads and
// are widened by the E4M3 conversion instruction (two codes per instruction).
// The row scales are read like the mask, one per lane for each 64-row block of the
// split, and a row's scale is taken from the lane that holds it: the K scale
// multiplies the row's score, the V scale its weight in O (the sum of weights
// uses the unscaled weight).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8_fp8(const u32x2_t& w, float (&f)[8]) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const f2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[0], false);
  const f2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[0], true);
  const f2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[1], false);
  const f2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[1], true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// Code formats of the static split pass: the word one lane loads for its 8
// elements of a row, how a row's bytes shrink (row bytes = D / kRowDiv), and the
// widening to fp32.
struct E4M3Rows {                          // one byte per element
  typedef u32x2_t Word;
  static constexpr int kRowDiv = 1;
  __device__ static Word load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLoadNonTemporal);
  }
  __device__ static void unpack(const Word& w, float (&f)[8]) { unpack8_fp8(w, f); }
  __device__ static Word select(bool ok, const Word& w) {   // w, or the +0 codes
    return Word{ok ? w[0] : 0u, ok ? w[1] : 0u};
  }
  // the scale exponent of a row with largest magnitude amax, and 8 values' codes
  __device__ static int exponent_for(float amax) { return e4m3_exponent_for(amax); }
  __device__ static Word quantise8(const float (&x)[8], int e) {
    Word w = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_code(ldexpf(x[i], -e)) << (8 * (i & 3));
    return w;
  }
};

struct E2M1Rows {                          // half a byte per element, element 2i low
  typedef uint32_t Word;
  static constexpr int kRowDiv = 2;
  __device__ static Word load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kLoadNonTemporal);
  }
  __device__ static void unpack(const Word& w, float (&f)[8]) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    const f2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 0);
    const f2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 1);
    const f2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 2);
    const f2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 3);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
  }
  __device__ static Word select(bool ok, const Word& w) { return ok ? w : 0u; }
  __device__ static int exponent_for(float amax) { return e2m1_exponent_for(amax); }
  __device__ static Word quantise8(const float (&x)[8], int e) {
    Word w = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(ldexpf(x[i], -e)) << (4 * i);
    return w;
  }
};

//
// The same pass serves the FP4 cache (Fmt = E2M1Rows, 4-byte loads).  With
// kAppend (decode_step_static_fp8 / _fp4) the split that owns p = write_pos[b]
// quantises the new token's K and V rows (as kv_append_fp8 / kv_append_fp4 do) in
// the lanes that later consume row p, once their first loads are issued; they
// store codes and scales and keep both in registers for that row, and p is
// attended whatever its mask entry says.
// Occupancy: at one or two steps the kernel fits 7 waves per SIMD (<= 72 VGPRs);
// left to itself the append variant takes 73 and drops to 6 (the fused batch-8
// call measured 32.8 us at 6 waves, 31.4 us at 7).
template <typename Fmt, int D, int U, int kSteps, bool kAppend>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kSteps <= 2 ? 7 : 3)))
static_decode_lowbit_kernel(const float* __restrict__ q, uint8_t* __restrict__ k_codes,
                         uint8_t* __restrict__ v_codes, float* __restrict__ k_scale,
                         float* __restrict__ v_scale, int32_t* __restrict__ mask,
                         const int32_t* __restrict__ valid_len, const uint16_t* __restrict__ k_new,
                         const uint16_t* __restrict__ v_new, const int32_t* __restrict__ write_pos,
                         int H, int cap, float scale_log2, int chunk, int units, Workspace ws,
                         float* __restrict__ out, float* __restrict__ lse, int32_t* err_flag) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int kStep = kWaves * RPW * U;             // rows per step
  constexpr int kBallots = (kSteps * kStep + 63) / 64;
  // the rows a wave loads at once (kWaves * RPW per u) tile 64-row words, so a
  // lane group's row never leaves the word (s kStep + u kWaves RPW) / 64
  static_assert(64 % (kWaves * RPW) == 0, "row words");
  constexpr int kRowBytes = D / Fmt::kRowDiv;
  typedef typename Fmt::Word Word;
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
  const float* ksrow = k_scale + (size_t)bh * cap;
  const float* vsrow = v_scale + (size_t)bh * cap;
  // before any wait: the valid length, the append position, the query and, per
  // 64-row block of the split, the mask entry of row r0 + 64 k + lane (clamped).
  // The row scales are first used after the codes arrive, so they go out only
  // once the split is known to hold rows.
  const int Lraw = valid_len ? valid_len[b] : cap;
  int p = kAppend ? write_pos[b] : -1;
  const float4* qp = reinterpret_cast<const float4*>(q + (size_t)bh * D + sub * 8);
  const float4 qa = qp[0], qc = qp[1];
  // (loaded under one uniform branch and tested at the ballots: a per-entry select
  // would make each load wait for the one before it)
  int32_t mv[kBallots];
  if (mrow) {
#pragma unroll
    for (int k = 0; k < kBallots; ++k) mv[k] = mrow[min(r0 + 64 * k + lane, cap - 1)];
  }
  const bool report = split == 0 && h == 0 && threadIdx.x == 0;
  // the appended row's codes and scales, in the lanes that own it.  E4M3: its bf16
  // rows are loaded here but quantised and stored only once this wave's first
  // code loads are in flight (the row enters the attention from registers, so
  // nothing waits for those stores): the owning splits are the last ones of their
  // heads, dispatched late, and the quantiser ahead of their loads cost the fused
  // batch-8 step 2% (977 against 958 us per step).  E2M1 quantises at once (late,
  // its step measured 1% slower).
  constexpr bool kLate = Fmt::kRowDiv == 1;
  float new_ks = 0.f, new_vs = 0.f;
  Word new_kw{}, new_vw{};
  bool owner = false;
  uint4 kn{}, vn{};
  auto append = [&]() {
    float kx[8], vx[8];
    unpack8(kn, kx);
    unpack8(vn, vx);
    float ka = 0.f, va = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ka = fmaxf(ka, fabsf(kx[i]));
      va = fmaxf(va, fabsf(vx[i]));
    }
    ka = group_max<LPR>(ka);
    va = group_max<LPR>(va);
    const int ke = Fmt::exponent_for(ka), ve = Fmt::exponent_for(va);
    const Word kw = Fmt::quantise8(kx, ke), vw = Fmt::quantise8(vx, ve);
    const size_t at = (((size_t)bh * cap + p) * D + (size_t)sub * 8) / Fmt::kRowDiv;
    *reinterpret_cast<Word*>(k_codes + at) = kw;
    *reinterpret_cast<Word*>(v_codes + at) = vw;
    new_kw = kw;
    new_vw = vw;
    new_ks = ldexpf(1.f, ke);
    new_vs = ldexpf(1.f, ve);
    if (sub == 0) {
      k_scale[(size_t)bh * cap + p] = new_ks;
      v_scale[(size_t)bh * cap + p] = new_vs;
    }
  };
  if constexpr (kAppend) {
    if (p < 0 || p >= cap) {
      if (report) raise_flag(err_flag, 2);
      p = -1;
    } else if (p / chunk == split) {
      const int o = p - r0;
      owner = wave == (o / RPW) % kWaves && slot == o % RPW;
      if (owner) {
        kn = load16(k_new + (size_t)bh * D + sub * 8);
        vn = load16(v_new + (size_t)bh * D + sub * 8);
        if constexpr (!kLate) append();
      }
      if (mask && h == 0 && threadIdx.x == 0) mask[(size_t)b * cap + p] = 1;
    } else {
      p = -1;  // another split holds the new row
    }
  }
  int L = Lraw;
  if (L < 0 || L > cap) {
    if (report) raise_flag(err_flag, 16);
    L = L < 0 ? 0 : cap;
  }
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  if (split >= n) {
    if (kAppend && kLate && owner) append();  // a row past the attended ones is still stored
    return;
  }
  // scales of the split's rows (row p's, if this split stores it, is taken from the
  // quantiser below, not from memory)
  float ksv[kBallots], vsv[kBallots];
#pragma unroll
  for (int k = 0; k < kBallots; ++k) {
    const int r = min(r0 + 64 * k + lane, cap - 1);
    ksv[k] = ksrow[r];
    vsv[k] = vsrow[r];
  }
  const int r1 = min(r0 + chunk, L);
  float qr[8];
  qr[0] = qa.x * scale_log2; qr[1] = qa.y * scale_log2;
  qr[2] = qa.z * scale_log2; qr[3] = qa.w * scale_log2;
  qr[4] = qc.x * scale_log2; qr[5] = qc.y * scale_log2;
  qr[6] = qc.z * scale_log2; qr[7] = qc.w * scale_log2;
  uint64_t bits[kBallots];
#pragma unroll
  for (int k = 0; k < kBallots; ++k)
    bits[k] = __ballot(r0 + 64 * k + lane < r1 && (!mrow || mv[k] != 0));
  const __amdgpu_buffer_rsrc_t kr_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(k_codes) + (size_t)bh * cap * kRowBytes, (short)0, cap * kRowBytes,
      0x00020000);
  const __amdgpu_buffer_rsrc_t vr_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(v_codes) + (size_t)bh * cap * kRowBytes, (short)0, cap * kRowBytes,
      0x00020000);
  const uint32_t lane_off = (uint32_t)sub * (8 / Fmt::kRowDiv);
  float m = kNegInf, l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  // rows of step s for this lane group: t = r0 + s kStep + (u kWaves + wave) RPW + slot
  auto issue = [&](int s, Word (&kw)[U], Word (&vw)[U], bool (&ok)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o_row = s * kStep + (u * kWaves + wave) * RPW + slot;  // row - r0
      const int word = (s * kStep + u * kWaves * RPW) >> 6;            // == o_row >> 6
      ok[u] = r0 + o_row < r1 &&
              (((bits[word] >> (o_row - 64 * word)) & 1ull) || r0 + o_row == p);
      const uint32_t off =
          ok[u] ? (uint32_t)(r0 + o_row) * kRowBytes + lane_off : BufferRows::kNoRow;
      kw[u] = Fmt::load(kr_rs, off);
      vw[u] = Fmt::load(vr_rs, off);
    }
  };
  auto consume = [&](int s, const Word (&kw)[U], const Word (&vw)[U], const bool (&ok)[U]) {
    float sc[U], ws_v[U];
    bool fresh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o_row = s * kStep + (u * kWaves + wave) * RPW + slot;
      // the appended row comes from registers, never from a load that follows
      // this lane's own store
      fresh[u] = kAppend && r0 + o_row == p;
      float kf[8];
      Word kcur = kw[u];
      if constexpr (kAppend) kcur = fresh[u] ? new_kw : kcur;
      Fmt::unpack(kcur, kf);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(qr[i], kf[i], acc);
      acc = group_sum<LPR>(acc);
      const int word = (s * kStep + u * kWaves * RPW) >> 6;            // == o_row >> 6
      // both shuffles run in every lane (a lane reads another lane's scale, so
      // none may sit out), then the appended row takes its own
      const float ksh = __shfl(ksv[word], o_row - 64 * word);
      const float vsh = __shfl(vsv[word], o_row - 64 * word);
      const float ks = fresh[u] ? new_ks : ksh;
      // a row that is not attended has zero codes (its load is past the resource)
      // and gets weight 0; its stored V scale may be anything, an infinity or NaN
      // included, so the scale it enters O with is 0, not the stored one
      ws_v[u] = ok[u] ? (fresh[u] ? new_vs : vsh) : 0.f;
      sc[u] = ok[u] ? acc * ks : kNegInf;
    }
    float mnew = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, sc[u]);
    const float ms = mnew == kNegInf ? 0.f : mnew;
    const float alpha = exp2_fast(m - ms);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    m = mnew;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2_fast(sc[u] - ms);
      l += p;
      const float pv = p * ws_v[u];
      float vf[8];
      Word vcur = vw[u];
      if constexpr (kAppend) vcur = fresh[u] ? new_vw : vcur;
      Fmt::unpack(vcur, vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(pv, vf[i], o[i]);
    }
  };
  Word kw[2][U], vw[2][U];
  bool ok[2][U];
  issue(0, kw[0], vw[0], ok[0]);
  if constexpr (kAppend && kLate) {
    if (owner) append();  // the first step's loads are in flight
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s + 1 < kSteps) issue(s + 1, kw[(s + 1) & 1], vw[(s + 1) & 1], ok[(s + 1) & 1]);
    consume(s, kw[s & 1], vw[s & 1], ok[s & 1]);
  }
  HeadState<1> st;
  st.m[0] = m;
  st.l[0] = l;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[0][i] = o[i];
  finish_split_flat<D>(st, lane, wave, ws, (size_t)bh, split, n, max_splits, out, lse);
}

template <typename Fmt, int D, int kSteps>
static void launch_static_fp8_k(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, int32_t* mask, const int32_t* valid_len,
                                const void* k_new, const void* v_new, const int32_t* write_pos,
                                int B, int H, int cap, float scale, float* out, float* lse,
                                const Workspace& w, const SplitPlan& plan, int32_t* err_flag,
                                hipStream_t stream) {
  const dim3 grid((unsigned)(B * H * plan.max_splits));
  auto* kc = static_cast<uint8_t*>(k_codes);
  auto* vc = static_cast<uint8_t*>(v_codes);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  if (write_pos) {
    hipLaunchKernelGGL((static_decode_lowbit_kernel<Fmt, D, 4, kSteps, true>), grid,
                       dim3(kThreads), 0, stream, q, kc, vc, k_scale, v_scale, mask, valid_len,
                       kn, vn, write_pos, H, cap, scale * kLog2e, plan.chunk, B * H, w, out,
                       lse, err_flag);
    return;
  }
  hipLaunchKernelGGL((static_decode_lowbit_kernel<Fmt, D, 4, kSteps, false>), grid,
                     dim3(kThreads), 0, stream, q, kc, vc, k_scale, v_scale, mask, valid_len, kn,
                     vn, write_pos, H, cap, scale * kLog2e, plan.chunk, B * H, w, out, lse,
                     err_flag);
}

template <typename Fmt>
static hipError_t launch_static_lowbit(const float* q, void* k_codes, void* v_codes,
                                       float* k_scale, float* v_scale, int32_t* mask,
                                       const int32_t* valid_len, const void* k_new,
                                       const void* v_new, const int32_t* write_pos, int B, int H,
                                       int cap, int D, float scale, float* out, float* lse,
                                       void* ws, const SplitPlan& plan, int32_t* err_flag,
                                       hipStream_t stream) {
  const Workspace w = carve(ws, (size_t)B * H, plan.max_splits, D);
#define DAKV_LOWBIT(DD)                                                                       \
  do {                                                                                        \
    constexpr int kStep = kWaves * (64 / (DD / 8)) * 4;                                       \
    const int steps = (plan.chunk + kStep - 1) / kStep;                                       \
    if (steps <= 1)                                                                           \
      launch_static_fp8_k<Fmt, DD, 1>(q, k_codes, v_codes, k_scale, v_scale, mask, valid_len, \
                                      k_new, v_new, write_pos, B, H, cap, scale, out, lse, w, \
                                      plan, err_flag, stream);                                \
    else if (steps <= 2)                                                                      \
      launch_static_fp8_k<Fmt, DD, 2>(q, k_codes, v_codes, k_scale, v_scale, mask, valid_len, \
                                      k_new, v_new, write_pos, B, H, cap, scale, out, lse, w, \
                                      plan, err_flag, stream);                                \
    else                                                                                      \
      launch_static_fp8_k<Fmt, DD, 4>(q, k_codes, v_codes, k_scale, v_scale, mask, valid_len, \
                                      k_new, v_new, write_pos, B, H, cap, scale, out, lse, w, \
                                      plan, err_flag, stream);                                \
  } while (0)
  if (D == 128) DAKV_LOWBIT(128);
  else DAKV_LOWBIT(64);
#undef DAKV_LOWBIT
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.max_splits <= 1) return err;
  return launch_static_merge(w, B, H, D, plan.chunk, plan.max_splits, valid_len, cap, out, lse,
                             stream);
}

hipError_t launch_decode_static_fp8(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                    float* v_scale, int32_t* mask, const int32_t* valid_len,
                                    const void* k_new, const void* v_new,
                                    const int32_t* write_pos, int B, int H, int cap, int D,
                                    float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  return launch_static_lowbit<E4M3Rows>(q, k_codes, v_codes, k_scale, v_scale, mask, valid_len,
                                        k_new, v_new, write_pos, B, H, cap, D, scale, out, lse,
                                        ws, plan, err_flag, stream);
}

hipError_t launch_decode_static_fp4(const float* q, const void* k_codes, const void* v_codes,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* mask, const int32_t* valid_len, int B, int H,
                                    int cap, int D, float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag, hipStream_t stream) {
  return launch_static_lowbit<E2M1Rows>(
      q, const_cast<void*>(k_codes), const_cast<void*>(v_codes), const_cast<float*>(k_scale),
      const_cast<float*>(v_scale), const_cast<int32_t*>(mask), valid_len, nullptr, nullptr,
      nullptr, B, H, cap, D, scale, out, lse, ws, plan, err_flag, stream);
}

hipError_t launch_decode_step_static_fp4(const float* q, void* k_codes, void* v_codes,
                                         float* k_scale, float* v_scale, int32_t* mask,
                                         const int32_t* valid_len, const void* k_new,
                                         const void* v_new, const int32_t* write_pos, int B,
                                         int H, int cap, int D, float scale, float* out,
                                         float* lse, void* ws, const SplitPlan& plan,
                                         int32_t* err_flag, hipStream_t stream) {
  return launch_static_lowbit<E2M1Rows>(q, k_codes, v_codes, k_scale, v_scale, mask, valid_len,
                                        k_new, v_new, write_pos, B, H, cap, D, scale, out, lse,
                                        ws, plan, err_flag, stream);
}

// ---------------------------------------------------------------------------
// paged_append_fp8 / paged_append_fp4: the new token of sequence b is its last
// token (position len_b - 1, len_b = seq_lens[b+1] - seq_lens[b] counting it),
// placed through the block table like every other token: block
// block_tables[b][seq_offset[b] / bs + t / bs], slot t % bs.  One wave per
// (sequence, KV head, K or V), as kv_append_fp8 / kv_append_fp4.  A sequence of
// length 0 or a bad table entry sets an error bit (DAKV_ERR_SEQ_LENS,
// DAKV_ERR_BLOCK_ID) and writes nothing.
// ---------------------------------------------------------------------------
template <bool kFp4>
__global__ void __launch_bounds__(256)
paged_append_lowbit_kernel(uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes,
                        float* __restrict__ k_scale, float* __restrict__ v_scale,
                        const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                        const int32_t* __restrict__ block_tables, int table_cols,
                        const int32_t* __restrict__ seq_lens,
                        const int32_t* __restrict__ seq_offset, int Hkv, int D, int num_blocks,
                        int block_size, int32_t* err_flag) {
  const int b = blockIdx.y;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);  // (head, K or V)
  const int lane = threadIdx.x & 63;
  if (unit >= 2 * Hkv) return;
  const int h = unit >> 1;
  const bool is_v = unit & 1;
  const bool report = unit == 0 && lane == 0;
  const int len = seq_lens[b + 1] - seq_lens[b];
  const int off = seq_offset ? seq_offset[b] : 0;
  if (len <= 0 || off < 0 || off % block_size != 0) {
    if (report) raise_flag(err_flag, 8);
    return;
  }
  const int t = len - 1;
  const int col = off / block_size + t / block_size;
  if (col >= table_cols) {
    if (report) raise_flag(err_flag, 8);
    return;
  }
  const int phys = block_tables[(size_t)b * table_cols + col];
  if (phys < 0 || phys >= num_blocks) {
    if (report) raise_flag(err_flag, 1);
    return;
  }
  const size_t row = ((size_t)phys * block_size + t % block_size) * Hkv + h;
  const uint16_t* src = (is_v ? v_new : k_new) + ((size_t)b * Hkv + h) * D;
  float* dscale = (is_v ? v_scale : k_scale) + row;
  if constexpr (kFp4)
    quantise_row_wave_fp4<2>(src, D, (is_v ? v_codes : k_codes) + row * (D / 2), dscale, lane);
  else
    quantise_row_wave<4>(src, D, (is_v ? v_codes : k_codes) + row * D, dscale, lane);
}

hipError_t launch_paged_append_fp8(void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hkv, int D, int num_blocks, int block_size,
                                   int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(paged_append_lowbit_kernel<false>, dim3((2 * Hkv + 3) / 4, B), dim3(256), 0,
                     stream, static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes),
                     k_scale, v_scale, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), block_tables, table_cols, seq_lens,
                     seq_offset, Hkv, D, num_blocks, block_size, err_flag);
  return hipGetLastError();
}

hipError_t launch_paged_append_fp4(void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hkv, int D, int num_blocks, int block_size,
                                   int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(paged_append_lowbit_kernel<true>, dim3((2 * Hkv + 3) / 4, B), dim3(256), 0,
                     stream, static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes),
                     k_scale, v_scale, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), block_tables, table_cols, seq_lens,
                     seq_offset, Hkv, D, num_blocks, block_size, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Paged GQA decode over the FP8 or FP4 pool: paged_rows_kernel's work split (one
// workgroup per (sequence, split) over all KV heads; lane group gi serves KV head
// gi % Hkv at token slot gi / Hkv) with 8 codes per lane (8 bytes of E4M3 or 4
// bytes of E2M1) and a row's K and V scales read by its lane group (one 4-byte
// address for the 16 lanes).  The K scale multiplies the row's scores, the V scale
// its weight in O.
// ---------------------------------------------------------------------------
// Step shape over the FP8 pool (rows per lane group per step, steps per unrolled
// super-step).  Measured at G = 4 (batch 64, block 16): U = 4 in one step 262 us,
// the bf16 kernel's 2 x 4 steps 318 us (178 VGPRs: 2 waves per SIMD), 2 x 2
// 291 us, 8 x 1 290 us; the other group sizes keep the bf16 shape.
template <int G> struct PagedShapeFp8 : PagedShape<G> {};
template <> struct PagedShapeFp8<4> { static constexpr int U = 4, kSteps = 1; };

template <typename Fmt, int G>
__global__ void __launch_bounds__(kThreads)
paged_rows_lowbit_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes,
                      const uint8_t* __restrict__ v_codes, const float* __restrict__ k_scale,
                      const float* __restrict__ v_scale, const int32_t* __restrict__ block_tables,
                      int table_cols, const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ seq_offset, int Hkv, int num_blocks,
                      int block_size, int bs_log2, int max_len, float scale_log2, int chunk,
                      int max_splits, Workspace ws, float* __restrict__ out,
                      float* __restrict__ lse, int32_t* err_flag) {
  constexpr int D = 128;
  constexpr int LPR = D / 8;
  constexpr int U = PagedShapeFp8<G>::U;
  constexpr int kSteps = PagedShapeFp8<G>::kSteps;
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
  const int bs_mask = block_size - 1;
  const size_t code_off = ((size_t)h * D + (size_t)sub * 8) / Fmt::kRowDiv;
  // the pool row (block, slot) of token t, or 0 with ok cleared (an in-bounds dummy)
  auto row_at = [&](int t, bool& ok) -> size_t {
    const int phys = ok ? tbl[(t >> bs_log2) - blk0] : -1;
    ok = phys >= 0;
    return ok ? (size_t)phys * block_size + (t & bs_mask) : 0;
  };
  typedef typename Fmt::Word Word;
  auto issue = [&](int t0, Word (&kw)[U], Word (&vw)[U], float (&ksc)[U],
                   float (&vsc)[U], bool (&ok)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * ts;
      ok[u] = t < r1;
      const size_t row = row_at(t, ok[u]);
      const size_t c = row * Hkv * (D / Fmt::kRowDiv) + code_off;
      kw[u] = __builtin_nontemporal_load(reinterpret_cast<const Word*>(k_codes + c));
      const Word v_in = __builtin_nontemporal_load(reinterpret_cast<const Word*>(v_codes + c));
      ksc[u] = k_scale[row * Hkv + h];
      const float vs_in = v_scale[row * Hkv + h];
      // an unused row re-reads pool row 0, which may hold NaN codes or scales: its V
      // codes (0 is the +0 code) and V scale become zeros once they arrive, so it
      // adds exactly nothing to O; its score is replaced by -inf below
      vw[u] = Fmt::select(ok[u], v_in);
      vsc[u] = ok[u] ? vs_in : 0.f;
    }
  };
  HeadState<G> st;
  init_state(st);
  auto consume = [&](const Word (&kw)[U], const Word (&vw)[U], const float (&ksc)[U],
                     const float (&vsc)[U], const bool (&ok)[U]) {
    float s[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      Fmt::unpack(kw[u], kf);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(qr[j][i], kf[i], acc);
        acc = group_sum<LPR>(acc);
        s[j][u] = ok[u] ? acc * ksc[u] : kNegInf;
      }
    }
    float vf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) Fmt::unpack(vw[u], vf[u]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mnew = st.m[j];
#pragma unroll
      for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, s[j][u]);
      const float ms = mnew == kNegInf ? 0.f : mnew;
      const float alpha = exp2_fast(st.m[j] - ms);
      float psum = 0.f;
      float pw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2_fast(s[j][u] - ms);
        psum += p;
        pw[u] = p * vsc[u];
      }
      st.l[j] = fmaf(st.l[j], alpha, psum);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.o[j][i] *= alpha;
      st.m[j] = mnew;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st.o[j][i] = fmaf(pw[u], vf[u][i], st.o[j][i]);
      }
    }
  };
  const int step = U * ts;
  const int super = step * kSteps;
  for (int base = r0; base < r1; base += super) {
    Word kw[2][U], vw[2][U];
    float ksc[2][U], vsc[2][U];
    bool ok[2][U];
    issue(base + slot, kw[0], vw[0], ksc[0], vsc[0], ok[0]);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + 1 < kSteps)
        issue(base + slot + (s + 1) * step, kw[(s + 1) & 1], vw[(s + 1) & 1], ksc[(s + 1) & 1],
              vsc[(s + 1) & 1], ok[(s + 1) & 1]);
      consume(kw[s & 1], vw[s & 1], ksc[s & 1], vsc[s & 1], ok[s & 1]);
    }
  }
  finish_split_rows<G>(st, gi, sub, Hkv, ts, ws, (size_t)b * Hq, split, n, max_splits, out, lse);
}

template <typename Fmt>
static hipError_t launch_paged_lowbit(const void* q, const void* k_codes, const void* v_codes,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_tables, int table_cols,
                                      const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                      int Hq, int Hkv, int num_blocks, int block_size,
                                      int max_seq_len, float scale, float* out, float* lse,
                                      void* ws, const SplitPlan& plan, int32_t* err_flag,
                                      hipStream_t stream) {
  const Workspace w = carve(ws, (size_t)B * Hq, plan.max_splits, 128);
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint8_t*>(k_codes);
  const auto* vc = static_cast<const uint8_t*>(v_codes);
  const dim3 grid((unsigned)(B * plan.max_splits));
#define DAKV_PAGED_FP8(GG)                                                                    \
  hipLaunchKernelGGL((paged_rows_lowbit_kernel<Fmt, GG>), grid, dim3(kThreads), 0, stream, qb, kc, vc, \
                     k_scale, v_scale, block_tables, table_cols, seq_lens, seq_offset, Hkv,  \
                     num_blocks, block_size, bs_log2, max_seq_len, scale * kLog2e,           \
                     plan.chunk, plan.max_splits, w, out, lse, err_flag)
  switch (Hq / Hkv) {
    case 1: DAKV_PAGED_FP8(1); break;
    case 2: DAKV_PAGED_FP8(2); break;
    case 4: DAKV_PAGED_FP8(4); break;
    case 8: DAKV_PAGED_FP8(8); break;
    default: return hipErrorInvalidValue;
  }
#undef DAKV_PAGED_FP8
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.max_splits <= 1) return err;
  return launch_paged_merge(w, B, Hq, plan.chunk, plan.max_splits, seq_lens, seq_offset,
                            block_size, table_cols, max_seq_len, out, lse, stream);
}

hipError_t launch_decode_paged_fp8(const void* q, const void* k_codes, const void* v_codes,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hq, int Hkv, int num_blocks, int block_size,
                                   int max_seq_len, float scale, float* out, float* lse,
                                   void* ws, const SplitPlan& plan, int32_t* err_flag,
                                   hipStream_t stream) {
  return launch_paged_lowbit<E4M3Rows>(q, k_codes, v_codes, k_scale, v_scale, block_tables,
                                       table_cols, seq_lens, seq_offset, B, Hq, Hkv, num_blocks,
                                       block_size, max_seq_len, scale, out, lse, ws, plan,
                                       err_flag, stream);
}

hipError_t launch_decode_paged_fp4(const void* q, const void* k_codes, const void* v_codes,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hq, int Hkv, int num_blocks, int block_size,
                                   int max_seq_len, float scale, float* out, float* lse,
                                   void* ws, const SplitPlan& plan, int32_t* err_flag,
                                   hipStream_t stream) {
  return launch_paged_lowbit<E2M1Rows>(q, k_codes, v_codes, k_scale, v_scale, block_tables,
                                       table_cols, seq_lens, seq_offset, B, Hq, Hkv, num_blocks,
                                       block_size, max_seq_len, scale, out, lse, ws, plan,
                                       err_flag, stream);
}

}  // namespace dakv
