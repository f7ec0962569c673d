// Streaming HBM read probe: a measurement utility beside the attention path
// (it gives the practical read ceiling that the attention kernels' KV
// streams are compared with), not a step of the method. Every thread reads
// 16-byte chunks with the non-temporal hint, sixteen loads in flight per loop
// trip (4 KB per wave), and folds them with XOR so that no load can be
// dropped; each block writes the XOR of its words.
#include "device_common.hpp"
#include "internal.hpp"

namespace skv {
namespace {

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(256) void hbm_probe_kernel(const u32x4_t* buf, int64_t n16, uint32_t* out) {
  __shared__ uint32_t part[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  constexpr int kU = 16;   // loads in flight per thread and trip
  for (; i + (kU - 1) * stride < n16; i += kU * stride) {
    u32x4_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(buf + i));
  // XOR over the block: within each wave by lane exchanges, then across waves
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_hbm_probe(const void* buf, int64_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(buf), bytes / 16, out);
  return hipGetLastError();
}


// Matrix-core and mixed-load probe: a measurement utility beside the
// attention path, like the read probe above. The first `mfma_waves` waves of
// each work-group keep eight independent bf16 v_mfma_f32_16x16x32 chains busy
// for `iters` trips; their eight A operands differ from one product to the
// next and hold pseudo-random bf16 values (signs, exponents 2^-3..2^0, full
// mantissas), so the multipliers see changing data as they do under
// attention. The other waves of the work-group stream `passes` passes over a
// buffer with the non-temporal hint (16 loads of 16 bytes in flight per lane),
// so that a launch can put the products and an HBM stream on the chip at the
// same time, in any proportion. It states the bf16 product rate the chip
// sustains under a dense matrix load alone, and what a launch that does
// nothing but products and a stream reaches at a given flop-per-byte ratio
// (power and clock included): the ceilings beside which a matrix-side
// attention launch is read. Per wave it writes a word folded from its results
// (so no product or load is dropped) and the shader-clock cycles it took.
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // a 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// Two bf16 values from a hash: sign, exponent 124..127, seven mantissa bits.
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  const uint32_t lo = (h & 0x807Fu) | ((124u + ((h >> 7) & 3u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807Fu) | ((124u + ((h >> 23) & 3u)) << 7);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(512) void mfma_probe_kernel(const u32x4_t* buf, int64_t n16, int passes, int iters,
                                                         int mfma_waves, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const uint32_t wid = blockIdx.x * wpb + wave;
  uint32_t res;
  uint64_t t0, t1;
  if (wave < mfma_waves) {
    u32x4_t a[8], b[2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[j][e] = rand_bf16x2(mix32((wid * 64 + lane) * 64 + 4 * j + e));
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) b[j][e] = rand_bf16x2(mix32(0x9e3779b9u ^ ((wid * 64 + lane) * 8 + 4 * j + e)));
    f32x4_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[j]),
                                                       __builtin_bit_cast(bf16x8_t, b[j & 1]), c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    t1 = __builtin_amdgcn_s_memtime();
    res = __float_as_uint(s);   // lane 0's value is the one written
  } else {
    // the streaming waves of the grid read the buffer grid-stride, lane by lane
    const int sw = wpb - mfma_waves;
    const int64_t nthreads = (int64_t)gridDim.x * sw * 64;
    const int64_t tid = ((int64_t)blockIdx.x * sw + (wave - mfma_waves)) * 64 + lane;
    uint32_t acc = 0;
    t0 = __builtin_amdgcn_s_memtime();
    for (int p = 0; p < passes; ++p) {
      int64_t i = tid;
      constexpr int kU = 16;
      for (; i + (kU - 1) * nthreads < n16; i += kU * nthreads) {
        u32x4_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * nthreads);
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
      }
      for (; i < n16; i += nthreads) {
        const u32x4_t v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
    t1 = __builtin_amdgcn_s_memtime();
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    res = acc;
  }
  if (lane == 0) {
    out[2 * wid] = res;
    out[2 * wid + 1] = (uint32_t)(t1 - t0);
  }
}

}  // namespace

hipError_t launch_mfma_probe(const void* buf, int64_t bytes, int passes, int blocks, int waves, int mfma_waves,
                             int iters, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(64 * waves), 0, stream,
                     static_cast<const u32x4_t*>(buf), bytes / 16, passes, iters, mfma_waves, out);
  return hipGetLastError();
}

}  // namespace skv
