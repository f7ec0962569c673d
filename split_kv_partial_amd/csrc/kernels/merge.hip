// Exact LSE merge of partial attention states (LiquidCP section 3, Equation 1:
// o = sum_r exp(lse_r) o_r / sum_r exp(lse_r); the Helix deep dive rescales each
// partial by exp(lse_r - lse_global) and sums). Each wave merges one unit: a run
// of consecutive output rows of one request. For a row, lane k holds the LSE of
// state k (the request's local splits first, then the external states), the
// wave forms M = max lse, w_k = exp(lse_k - M) and Z = sum w_k, and then streams
// the states' output vectors with lanes across the value dimension, skipping
// states of zero weight. The kernel is a pure HBM stream: every state vector is
// read once, coalesced, and every output row written once.
#include "device_common.hpp"
#include "internal.hpp"

namespace skv {

struct MergeArgs {
  const DevReq* reqs;
  const DevUnit* units;
  const float* o_part;
  const float* lse_part;
  const float* o_ext;
  const float* lse_ext;
  void* o_out;
  float* lse_out;
  int64_t total_rows;
  int32_t n_ext, num_units, out_bf16;
};

template <int DV>
struct VecIO;
template <>
struct VecIO<64> {  // one float per lane
  static constexpr int N = 1;
  __device__ static void load(const float* p, int lane, float* v) { v[0] = __builtin_nontemporal_load(p + lane); }
};
template <>
struct VecIO<128> {  // two floats per lane
  static constexpr int N = 2;
  __device__ static void load(const float* p, int lane, float* v) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const f32x2v x = __builtin_nontemporal_load(reinterpret_cast<const f32x2v*>(p) + lane);
    v[0] = x[0];
    v[1] = x[1];
  }
};
template <>
struct VecIO<512> {  // eight floats per lane: dims 4l..4l+3 and 256+4l..256+4l+3
  static constexpr int N = 8;
  __device__ static void load(const float* p, int lane, float* v) {
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + lane);
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 256) + lane);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  }
};

// Dimension held in slot i of lane `lane` (matches VecIO::load).
template <int DV>
__device__ __forceinline__ int dim_of(int lane, int i) {
  if constexpr (DV == 64) return lane;
  if constexpr (DV == 128) return 2 * lane + i;
  return (i < 4 ? 0 : 256) + 4 * lane + (i & 3);
}

template <int DV>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int N = VecIO<DV>::N;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.num_units) return;
  const DevUnit u = a.units[unit];
  const DevReq rq = a.reqs[u.b];
  const int S = rq.splits + a.n_ext;  // <= 64 + n_ext, at most 128 (host-checked)

  for (int r = u.row; r < u.row + u.count; ++r) {
    const int64_t out_row = (int64_t)rq.out_row + r;
    auto lse_of = [&](int k) -> float {
      if (k < rq.splits) return a.lse_part[(int64_t)rq.state_row + (int64_t)k * rq.rows + r];
      return a.lse_ext[(int64_t)(k - rq.splits) * a.total_rows + out_row];
    };
    auto src_of = [&](int k) -> const float* {
      return k < rq.splits ? a.o_part + ((int64_t)rq.state_row + (int64_t)k * rq.rows + r) * DV
                           : a.o_ext + ((int64_t)(k - rq.splits) * a.total_rows + out_row) * DV;
    };
    // Few states (the common decode case): fetch every state vector together
    // with the LSEs, so the row costs one memory round trip instead of two.
    constexpr int kFew = 8;
    float vf[kFew][N];
    if (S <= kFew) {
#pragma unroll
      for (int k = 0; k < kFew; ++k)
        if (k < S) VecIO<DV>::load(src_of(k), lane, vf[k]);
    }
    const float l0 = lane < S ? lse_of(lane) : -INFINITY;
    const float l1 = lane + 64 < S ? lse_of(lane + 64) : -INFINITY;
    const float M = wave_max(fmaxf(l0, l1));
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    float lse = -INFINITY;
    if (M != -INFINITY) {
      const float w0 = fast_exp2((l0 - M) * kLog2e);
      const float w1 = fast_exp2((l1 - M) * kLog2e);
      const float Z = wave_sum(w0 + w1);
      if (S <= kFew) {
#pragma unroll
        for (int k = 0; k < kFew; ++k) {
          if (k >= S) break;
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), k));
          // an empty state, or one negligible beyond fp32 range, takes no part
          // (its vector may hold anything, e.g. an external state's NaN)
#pragma unroll
          for (int i = 0; i < N; ++i) acc[i] = wk != 0.f ? fmaf(wk, vf[k][i], acc[i]) : acc[i];
        }
      } else {
        for (int k = 0; k < S; ++k) {
          const float wk = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(k < 64 ? w0 : w1), k & 63));
          if (wk == 0.f) continue;  // empty state, or negligible beyond fp32 range
          float v[N];
          VecIO<DV>::load(src_of(k), lane, v);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[i] = fmaf(wk, v[i], acc[i]);
        }
      }
      const float inv = 1.f / Z;
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] *= inv;
      lse = M + fast_log2(Z) * kLn2;
    }
    if (a.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(a.o_out) + out_row * DV;
#pragma unroll
      for (int i = 0; i < N; ++i) o[dim_of<DV>(lane, i)] = (uint16_t)f32_to_bf16_bits(acc[i]);
    } else {
      float* o = static_cast<float*>(a.o_out) + out_row * DV;
#pragma unroll
      for (int i = 0; i < N; ++i) o[dim_of<DV>(lane, i)] = acc[i];
    }
    if (a.lse_out && lane == 0) a.lse_out[out_row] = lse;
  }
}

hipError_t launch_merge(const MergeLaunch& m) {
  if (m.num_units == 0) return hipSuccess;
  MergeArgs a;
  const uint8_t* ws = static_cast<const uint8_t*>(m.workspace);
  a.reqs = reinterpret_cast<const DevReq*>(ws + m.reqs_off);
  a.units = reinterpret_cast<const DevUnit*>(ws + m.units_off);
  a.o_part = m.o_part;
  a.lse_part = m.lse_part;
  a.o_ext = m.o_ext;
  a.lse_ext = m.lse_ext;
  a.o_out = m.o_out;
  a.lse_out = m.lse_out;
  a.total_rows = m.total_rows;
  a.n_ext = m.n_ext;
  a.num_units = m.num_units;
  a.out_bf16 = m.out_bf16;
  const dim3 grid((m.num_units + 3) / 4), block(256);
  switch (m.head_dim_v) {
    case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, m.stream, a); break;
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, m.stream, a); break;
    case 512: hipLaunchKernelGGL(merge_kernel<512>, grid, block, 0, m.stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skv
