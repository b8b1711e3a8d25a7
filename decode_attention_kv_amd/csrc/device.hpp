// Device helpers shared by the gfx950 kernels: bf16 unpacking, 16-lane DPP
// reductions, the base-2 exponential, and the error-flag update.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dakv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Two bf16 values packed in one 32-bit word (element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 values of a 16-byte load as floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// v_exp_f32: 2^x, exact at 0, 0 at -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a row of 16 lanes.
//   0xB1 quad_perm [1,0,3,2]   (xor 1)
//   0x4E quad_perm [2,3,0,1]   (xor 2)
//   0x141 row_half_mirror      (lane i <- 7 - i within each 8)
//   0x140 row_mirror           (lane i <- 15 - i within each 16)
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum over aligned groups of kLanes lanes (kLanes in {4, 8, 16}); every lane of a
// group receives the group's sum.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  if constexpr (kLanes >= 8) v += dpp<0x141>(v);
  if constexpr (kLanes >= 16) v += dpp<0x140>(v);
  return v;
}

template <int kLanes>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (kLanes >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (kLanes >= 16) v = fmaxf(v, dpp<0x140>(v));
  return v;
}

__device__ __forceinline__ void raise_flag(int32_t* err_flag, int32_t bit) {
  if (err_flag) atomicOr(err_flag, bit);
}

// A store written through to the device's point of coherence (an agent-scope relaxed
// atomic store: cache policy sc1).  The persistent paged kernel writes its split
// partials this way as it goes: they do not sit dirty in the XCD's L2 among the streamed
// K/V lines until the end-of-kernel write-back (paged GQA call 262 -> 251 us).  Measured
// and not used elsewhere: the sparse pass, whose partials are all written at its end, is
// unchanged, and the static pass, whose short workgroups then end later, is slower (batch-8
// step 1294 -> 1382 us); so are the merge kernels' outputs (sparse call 34.0 -> 36.2 us,
// batch-8 step 1299 -> 1303 us).
__device__ __forceinline__ void store_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache-policy operand of a buffer store written through to the point of coherence
// (sc1).  A streaming copy that stores this way leaves no dirty lines in the XCD's L2
// (the paged gather: 87.5 -> 78.6 us per call, 494 MB moved; non-temporal stores, with
// or without sc1, measured the same as plain ones).
constexpr int kStoreThrough = 16;

// 16 bytes through a buffer resource with kStoreThrough
__device__ __forceinline__ void store16_through(__amdgpu_buffer_rsrc_t r, int off, const uint4& v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, kStoreThrough);
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void store16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// E4M3 quantisation of a row with a power-of-two scale 2^e: e is the smallest
// integer with amax <= 448 * 2^e (0 for amax = 0), from amax's exponent and
// fraction, exactly; a value y = x * 2^-e (|y| <= 448) gets the code of the
// nearest E4M3 value, ties to the even code, zero results as the +0 code.
__device__ __forceinline__ int e4m3_exponent_for(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);        // amax = f 2^E, f in [0.5, 1); 448 = 0.875 2^9
  return f <= 0.875f ? E - 9 : E - 8;
}

__device__ __forceinline__ uint32_t e4m3_code(float y) {  // |y| <= 448
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                     // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.f);     // 8 -> 2^-6, the smallest normal code
  } else {
    int F;
    const float f = frexpf(a, &F);         // a = (2f) 2^(F-1), 2f in [1, 2)
    uint32_t m = (uint32_t)rintf((2.f * f - 1.f) * 8.f);
    int E = F - 1;
    if (m == 8) {
      m = 0;
      ++E;
    }
    code = ((uint32_t)(E + 7) << 3) | m;
  }
  return (code != 0 && y < 0.f) ? (code | 0x80u) : code;
}

}  // namespace dakv
