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

}  // namespace skv
