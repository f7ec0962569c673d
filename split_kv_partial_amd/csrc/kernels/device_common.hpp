// Device-side helpers shared by the attention and merge kernels (gfx950, wave64).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace skv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device-side descriptor of one attention work-group (built by the host).
struct DevTask {
  int32_t b;        // request
  int32_t kvh;      // KV head
  int32_t lo;       // first KV token of the split (multiple of 64)
  int32_t end;      // one past the last KV token this task may read:
                    // min(split end, visible end of its query token)
  int32_t q_row;    // global query-token index
  int32_t out_row;  // state row of the task's first query head
  int32_t pad0, pad1;
};

struct DevReq {
  int32_t state_row, splits, rows, out_row;
};
struct DevUnit {
  int32_t b, row, count, pad;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (inputs here are finite or +-inf).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two-term bf16 representation of a softmax weight: p = hi + lo with hi the
// nearest bf16 and lo the nearest bf16 to the (exact) remainder, so hi + lo
// carries about 16 significant bits. Products with bf16 operands then lose
// ~2^-17 relative instead of the 2^-9 of a single bf16 rounding.
__device__ __forceinline__ void split_bf16(float p, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(p);
  lo = f32_to_bf16_bits(p - __uint_as_float(hi << 16));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Butterfly reductions over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Record a device error (vector atomic; bit 0 = page id outside the pool).
__device__ __forceinline__ void raise_error(int32_t* flag, int32_t bit) {
  atomicOr(flag, bit);
}

}  // namespace skv
