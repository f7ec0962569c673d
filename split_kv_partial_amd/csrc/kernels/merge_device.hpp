// Device side of the exact LSE merge of partial attention states (LiquidCP
// section 3, Equation 1: o = sum_r exp(lse_r) o_r / sum_r exp(lse_r); the Helix
// deep dive rescales each partial by exp(lse_r - lse_global) and sums), shared
// by the merge kernel and the fused attention-and-merge kernels. For a row,
// lane k holds the LSE of state k (the request's local splits first, then the
// external states), the wave forms M = max lse, w_k = exp(lse_k - M) and
// Z = sum w_k, and then streams the states' output vectors with lanes across
// the value dimension, skipping states of zero weight.
#pragma once

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

// Kernel arguments of a merge (host side).
inline MergeArgs merge_args(const MergeLaunch& m) {
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
  return a;
}

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

// How the merge reads a row's states. Plain: vector loads (the merge
// launch, whose inputs an earlier launch wrote). Coherent: the merge inside
// the fused launch reads partial states that other work-groups of the same
// launch wrote, possibly on another XCD, whose L2 this XCD's does not see:
// those loads are relaxed agent-scope atomic loads, which read the coherence
// point, one float per lane per instruction with slot i of lane l holding
// dimension 64 i + l (whole cache lines per instruction); external states,
// which the launch does not write, are plain loads in the same layout.
template <int DV, bool kCoherent>
struct StateIO {
  static constexpr int N = VecIO<DV>::N;
  __device__ static int dim(int lane, int i) { return kCoherent ? 64 * i + lane : dim_of<DV>(lane, i); }
  __device__ static void load_local(const float* p, int lane, float* v) {
    if constexpr (kCoherent) {
#pragma unroll
      for (int i = 0; i < N; ++i)
        v[i] = __hip_atomic_load(p + 64 * i + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      VecIO<DV>::load(p, lane, v);
    }
  }
  __device__ static void load_ext(const float* p, int lane, float* v) {
    if constexpr (kCoherent) {
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = __builtin_nontemporal_load(p + 64 * i + lane);
    } else {
      VecIO<DV>::load(p, lane, v);
    }
  }
  __device__ static float lse_local(const float* p) {
    if constexpr (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
  }
};

// The reference M = max of a row's state LSEs (lane k holds states k and
// k + 64). A NaN LSE marks a state its attention task could not compute (see
// the attention kernels' error flag): M is then NaN, so the whole merged row
// comes out NaN instead of the NaN being dropped by the maximum.
__device__ __forceinline__ float row_reference(float l0, float l1) {
  const float M = wave_max(fmaxf(l0, l1));
  return __builtin_amdgcn_ballot_w64(l0 != l0 || l1 != l1) != 0 ? __builtin_nanf("") : M;
}

constexpr int kFew = 8;   // states whose vectors are fetched together
constexpr int R = 8;      // rows per step of the many-state path

// Many states (external ones): R consecutive rows at a time, states in the
// outer loop. For a fixed state the R rows' vectors are contiguous, so a wave
// streams R x DV x 4 bytes from one or two states at a time instead of
// touching every state's stream for every row; each row still accumulates
// its states in state order, as the few-state path does. Measured on 263k
// rows x 17 states of 512 floats (MI355X): one wave per unit taking rows one
// at a time 1.98 ms -> R = 4: 1.79 -> R = 8 with two states in flight:
// 1.65 ms. The latter needs 268 registers (one wave per SIMD); trimmed to
// two waves per SIMD it ran slower (1.73 ms): fewer state streams at once
// per CU read faster.
template <int DV>
__device__ __forceinline__ void merge_rows_many(const MergeArgs& a, const DevUnit& u, const DevReq& rq,
                                                int S, int lane, int first, int stride) {
  constexpr int N = VecIO<DV>::N;
  constexpr int KB = 2;   // states per batch of loads: R x KB vectors in flight
  for (int r0 = u.row + first; r0 < u.row + u.count; r0 += stride) {
    const int nr = min(R, u.row + u.count - r0);
    auto lse_of = [&](int k, int r) -> float {
      if (k < rq.splits) return a.lse_part[(int64_t)rq.state_row + (int64_t)k * rq.rows + r];
      return a.lse_ext[(int64_t)(k - rq.splits) * a.total_rows + rq.out_row + r];
    };
    auto src_of = [&](int k, int r) -> const float* {
      return k < rq.splits ? a.o_part + ((int64_t)rq.state_row + (int64_t)k * rq.rows + r) * DV
                           : a.o_ext + ((int64_t)(k - rq.splits) * a.total_rows + rq.out_row + r) * DV;
    };
    float w0[R], w1[R], Z[R], M[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float l0 = j < nr && lane < S ? lse_of(lane, r0 + j) : -INFINITY;
      const float l1 = j < nr && lane + 64 < S ? lse_of(lane + 64, r0 + j) : -INFINITY;
      M[j] = row_reference(l0, l1);
      const bool live = M[j] != -INFINITY;
      w0[j] = live ? fast_exp2((l0 - M[j]) * kLog2e) : 0.f;
      w1[j] = live ? fast_exp2((l1 - M[j]) * kLog2e) : 0.f;
      Z[j] = wave_sum(w0[j] + w1[j]);
    }
    float acc[R][N];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[j][i] = 0.f;
    for (int k0 = 0; k0 < S; k0 += KB) {
      float wk[KB][R], v[KB][R][N];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = k0 + kb;
#pragma unroll
        for (int j = 0; j < R; ++j) {
          wk[kb][j] = k < S ? __int_as_float(__builtin_amdgcn_readlane(
                                  __float_as_int(k < 64 ? w0[j] : w1[j]), k & 63))
                            : 0.f;
          // an empty state, or one negligible beyond fp32 range, is not read
          // (its vector may hold anything, e.g. an external state's NaN)
          if (wk[kb][j] != 0.f) VecIO<DV>::load(src_of(k, r0 + j), lane, v[kb][j]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int i = 0; i < N; ++i)
            acc[j][i] = wk[kb][j] != 0.f ? fmaf(wk[kb][j], v[kb][j][i], acc[j][i]) : acc[j][i];
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j >= nr) break;
      const int64_t out_row = (int64_t)rq.out_row + r0 + j;
      float lse = -INFINITY;
      if (M[j] != -INFINITY) {
        const float inv = 1.f / Z[j];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[j][i] *= inv;
        lse = M[j] + fast_log2(Z[j]) * kLn2;
      }
      if (a.out_bf16) {
        uint16_t* o = static_cast<uint16_t*>(a.o_out) + out_row * DV;
#pragma unroll
        for (int i = 0; i < N; ++i) o[dim_of<DV>(lane, i)] = (uint16_t)f32_to_bf16_bits(acc[j][i]);
      } else {
        float* o = static_cast<float*>(a.o_out) + out_row * DV;
#pragma unroll
        for (int i = 0; i < N; ++i) o[dim_of<DV>(lane, i)] = acc[j][i];
      }
      if (a.lse_out && lane == 0) a.lse_out[out_row] = lse;
    }
  }
}

// One wave merges the rows of one unit, row by row: lane k holds the LSEs of
// states k and k + 64, the state vectors stream with lanes across D_v.
template <int DV, bool kCoherent = false>
__device__ __forceinline__ void merge_rows_wave(const MergeArgs& a, const DevUnit& u, const DevReq& rq,
                                                int S, int lane) {
  constexpr int N = VecIO<DV>::N;
  using IO = StateIO<DV, kCoherent>;
  for (int r = u.row; r < u.row + u.count; ++r) {
    const int64_t out_row = (int64_t)rq.out_row + r;
    auto lse_of = [&](int k) -> float {
      if (k < rq.splits) return IO::lse_local(a.lse_part + (int64_t)rq.state_row + (int64_t)k * rq.rows + r);
      return a.lse_ext[(int64_t)(k - rq.splits) * a.total_rows + out_row];
    };
    auto src_of = [&](int k) -> const float* {
      return k < rq.splits ? a.o_part + ((int64_t)rq.state_row + (int64_t)k * rq.rows + r) * DV
                           : a.o_ext + ((int64_t)(k - rq.splits) * a.total_rows + out_row) * DV;
    };
    auto load_state = [&](int k, float* v) {
      if (k < rq.splits) IO::load_local(src_of(k), lane, v);
      else IO::load_ext(src_of(k), lane, v);
    };
    // Few states (the common decode case): fetch every state vector together
    // with the LSEs, so the row costs one memory round trip instead of two.
    float vf[kFew][N];
    if (S <= kFew) {
#pragma unroll
      for (int k = 0; k < kFew; ++k)
        if (k < S) load_state(k, vf[k]);
    }
    const float l0 = lane < S ? lse_of(lane) : -INFINITY;
    const float l1 = lane + 64 < S ? lse_of(lane + 64) : -INFINITY;
    const float M = row_reference(l0, l1);
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
        // more states on a short unit: kFew vectors in flight per batch,
        // accumulated in state order
        for (int k0 = 0; k0 < S; k0 += kFew) {
          float wb[kFew];
#pragma unroll
          for (int j = 0; j < kFew; ++j) {
            const int k = k0 + j;
            wb[j] = k < S ? __int_as_float(
                                __builtin_amdgcn_readlane(__float_as_int(k < 64 ? w0 : w1), k & 63))
                          : 0.f;
            // an empty state, or one negligible beyond fp32 range, is not read
            if (wb[j] != 0.f) load_state(k, vf[j]);
          }
#pragma unroll
          for (int j = 0; j < kFew; ++j)
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] = wb[j] != 0.f ? fmaf(wb[j], vf[j][i], acc[i]) : acc[i];
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
      for (int i = 0; i < N; ++i) o[IO::dim(lane, i)] = (uint16_t)f32_to_bf16_bits(acc[i]);
    } else {
      float* o = static_cast<float*>(a.o_out) + out_row * DV;
#pragma unroll
      for (int i = 0; i < N; ++i) o[IO::dim(lane, i)] = acc[i];
    }
    if (a.lse_out && lane == 0) a.lse_out[out_row] = lse;
  }
}

// A unit whose inputs could not be waited for: its rows are written as NaN.
template <int DV>
__device__ __forceinline__ void merge_rows_nan(const MergeArgs& a, const DevUnit& u, const DevReq& rq,
                                               int lane) {
  const float nan = __builtin_nanf("");
  for (int r = u.row; r < u.row + u.count; ++r) {
    const int64_t out_row = (int64_t)rq.out_row + r;
    for (int d = lane; d < DV; d += 64) {
      if (a.out_bf16) static_cast<uint16_t*>(a.o_out)[out_row * DV + d] = 0x7FC0;
      else static_cast<float*>(a.o_out)[out_row * DV + d] = nan;
    }
    if (a.lse_out && lane == 0) a.lse_out[out_row] = nan;
  }
}

}  // namespace skv
