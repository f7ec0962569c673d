// Device-side helpers shared by the attention and merge kernels (gfx950, wave64).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace skv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (inputs here are finite or +-inf).
// fp32 -> bf16 with round-to-nearest-even (the gfx950 packed conversion
// instruction; NaN stays NaN).
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t{lo, hi}), bf16x2v_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// Two-term bf16 representation of a softmax weight: p = hi + lo with hi the
// nearest bf16 and lo the nearest bf16 to the (exact) remainder, so hi + lo
// carries about 16 significant bits. Products with bf16 operands then lose
// ~2^-17 relative instead of the 2^-9 of a single bf16 rounding.
__device__ __forceinline__ void split_bf16(float p, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(p);
  lo = f32_to_bf16_bits(p - __uint_as_float(hi << 16));
}
// The same split for a pair of weights, packed as two bf16x2 words.
__device__ __forceinline__ void split_bf16x2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(p0, p1);
  lo = pack_bf16x2(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Cross-lane reductions without LDS traffic. All 64 lanes must be active.
// DPP steps combine lanes within a 16-lane row (swap neighbours, swap pairs,
// mirror within 8, mirror within 16); the gfx950 lane-swap instructions then
// exchange whole rows (lane i with lane i^16, and lane i with lane i^32). Each
// step combines two values that every lane of the pair sees in the same
// order up to commutation, so the result is bit-identical in all lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

struct LanePair {
  float a, b;  // the lane's own value and its partner's, in lane-independent order
};
__device__ __forceinline__ LanePair pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor16(float v) {
  const LanePair p = pair16(v);
  return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float max_xor32(float v) {
  const LanePair p = pair32(v);
  return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const LanePair p = pair16(v);
  return p.a + p.b;
}
__device__ __forceinline__ float sum_xor32(float v) {
  const LanePair p = pair32(v);
  return p.a + p.b;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<kDppSwap1>(v));
  v = fmaxf(v, dpp_f<kDppSwap2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppSwap1>(v);
  v += dpp_f<kDppSwap2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
__device__ __forceinline__ float wave_max(float v) { return max_xor32(max_xor16(row_max16(v))); }
__device__ __forceinline__ float wave_sum(float v) { return sum_xor32(sum_xor16(row_sum16(v))); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Bits of the workspace's device error flag.
constexpr int32_t kErrPageId = 1;   // a page id outside [0, num_pages)
constexpr int32_t kErrSeqLen = 2;   // device seq_lens differ from the plan's
constexpr int32_t kErrRange = 4;    // scores beyond the range the softmax represents
constexpr int32_t kErrWait = 8;     // a merge gave up waiting for its inputs

// Record a device error (a vector atomic OR into the flag word).
__device__ __forceinline__ void raise_error(int32_t* flag, int32_t bit) {
  atomicOr(flag, bit);
}

// The state of a task that met an error: every thread of the work-group
// writes its share of rows [row0, row0 + nrows) of o (dv floats each) and lse
// as NaN, so that the merged rows of the task come out NaN as well.
__device__ __forceinline__ void write_nan_state(float* o, float* lse, int64_t row0, int nrows, int dv) {
  const float nan = __builtin_nanf("");
  for (int i = threadIdx.x; i < nrows * dv; i += blockDim.x) o[row0 * dv + i] = nan;
  for (int i = threadIdx.x; i < nrows; i += blockDim.x) lse[row0 + i] = nan;
}

}  // namespace skv
