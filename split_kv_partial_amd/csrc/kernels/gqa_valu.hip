// Paged split-KV partial attention on the vector ALUs for fp32 GQA (any group
// size up to 16) and bf16 groups of fewer than 8 query heads per KV head
// (fp32 accumulation); bf16 groups of 8 and 16 run on the matrix cores.
//
// One work-group (4 waves) runs one task: KV head g of one query token over
// the KV range [lo, end) of one split. The waves take the split's 64-token
// tiles round-robin, each keeping its own online-softmax state; the four
// states are merged through LDS at the end and written as the split's partial
// state (output normalised over the split, natural-log LSE; LiquidCP section
// 2.1 and Equation 1).
//
// Per tile, a wave computes scores with one lane per token (the key row of
// that token is one coalesced read of its 16-byte chunks, query values are
// LDS broadcasts), reduces the tile maximum across lanes, and then
// accumulates P*V with one lane per value dimension (values are stored
// dimension-major per page, so a lane reads its dimension's tokens as one
// contiguous run). bf16 products use the packed dot2 instruction; the softmax
// weights enter it as a two-term bf16 pair (hi + lo) so that P*V keeps ~16
// significant bits of each weight.
#include "device_common.hpp"
#include "fused.hpp"
#include "internal.hpp"

namespace skv {

struct ValuArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const DevTask* tasks;
  int32_t* err_flag;
  float* o_part;
  float* lse_part;
  int32_t H_q, H_kv, page_shift, max_pages, num_pages;
  float scale_log2;  // softmax scale * log2(e)
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int X = 4;  // elements per 16-byte chunk
};
template <>
struct Elem<uint16_t> {
  static constexpr int X = 8;
};

constexpr int kWaves = 4;
constexpr int kTile = 64;

// LDS of one work-group.
template <typename T, int D, int G>
struct ValuShared {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int QW = kBf16 ? D / 2 : D;  // 32-bit words per query row in LDS
  uint32_t q_lds[G * QW];
  // Softmax weights of the current tile, private to each wave: fp32, or bf16
  // (the bf16 path feeds them to dot2 in token pairs).
  float p_lds[kWaves][G][kBf16 ? 1 : kTile];
  uint16_t p16_lds[kWaves][2][G][kBf16 ? kTile : 2];   // [hi, lo]
  float m_lds[kWaves][G], l_lds[kWaves][G];
  float o_lds[kWaves][G][D];
  int bad_lds[kWaves];
};

// One task: KV head g of one query token over the KV range [lo, end) of one
// split, written as the split's partial state.
template <typename T, int D, int G>
__device__ __forceinline__ void gqa_valu_task(const ValuArgs& a, const DevTask& t, ValuShared<T, D, G>& sh) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int X = Elem<T>::X;
  constexpr int NC = D / X;          // 16-byte chunks per key row
  constexpr int DL = D / 64;         // value dimensions per lane
  constexpr int QW = kBf16 ? D / 2 : D;  // 32-bit words per query row in LDS
  auto& q_lds = sh.q_lds;
  auto& p_lds = sh.p_lds;
  auto& p16_lds = sh.p16_lds;
  auto& m_lds = sh.m_lds;
  auto& l_lds = sh.l_lds;
  auto& o_lds = sh.o_lds;
  auto& bad_lds = sh.bad_lds;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int P = 1 << a.page_shift;
  if (a.seq_lens[t.b] != t.seq_len) {
    // the device lengths are not the ones the plan was built from: no KV is
    // read and the state is NaN (uniform over the work-group: one task)
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrSeqLen);
    write_nan_state(a.o_part, a.lse_part, t.out_row, G, D);
    return;
  }
  const int end = t.end;
  bool bad = false;   // this lane met a page id outside the pool

  // Query rows of the G heads of this KV head into LDS (fp32 or packed bf16).
  {
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(
        static_cast<const T*>(a.q) + ((int64_t)t.q_row * a.H_q + (int64_t)t.kvh * G) * D);
    for (int i = threadIdx.x; i < G * QW; i += 256) q_lds[i] = qsrc[i];
  }
  __syncthreads();

  const int32_t* ptab = a.page_table + (int64_t)t.b * a.max_pages;
  float m[G], l[G], o[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < DL; ++k) o[h][k] = 0.f;
  }

  for (int tok0 = t.lo + wave * kTile; tok0 < end; tok0 += kWaves * kTile) {
    // ---------------- scores: one lane per token ----------------
    const int j = tok0 + lane;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    bool valid = j < end;
    if (valid) {
      const int pid = ptab[j >> a.page_shift];
      if (pid < 0 || pid >= a.num_pages) {   // not read; the state becomes NaN
        raise_error(a.err_flag, kErrPageId);
        bad = true;
        valid = false;
      } else {
        const uint8_t* kp = static_cast<const uint8_t*>(a.k) +
                            (((int64_t)pid * a.H_kv + t.kvh) * NC * P + (j & (P - 1))) * 16;
        u32x4_t kr[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
          kr[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + (int64_t)c * P * 16));
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(&q_lds[h * QW + c * 4]);
            if constexpr (kBf16) {
              s[h] = dot2_bf16(qv[0], kr[c][0], s[h]);
              s[h] = dot2_bf16(qv[1], kr[c][1], s[h]);
              s[h] = dot2_bf16(qv[2], kr[c][2], s[h]);
              s[h] = dot2_bf16(qv[3], kr[c][3], s[h]);
            } else {
              s[h] = fmaf(__uint_as_float(qv[0]), __uint_as_float(kr[c][0]), s[h]);
              s[h] = fmaf(__uint_as_float(qv[1]), __uint_as_float(kr[c][1]), s[h]);
              s[h] = fmaf(__uint_as_float(qv[2]), __uint_as_float(kr[c][2]), s[h]);
              s[h] = fmaf(__uint_as_float(qv[3]), __uint_as_float(kr[c][3]), s[h]);
            }
          }
        }
      }
    }
    // ---------------- online softmax (log2 domain) ----------------
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = valid ? s[h] * a.scale_log2 : -INFINITY;
      const float mt = wave_max(sv);
      const float mn = fmaxf(m[h], mt);
      alpha[h] = fast_exp2(m[h] - mn);  // m = -inf on the first tile gives 0
      m[h] = mn;
      const float p = fast_exp2(sv - mn);
      l[h] = l[h] * alpha[h] + p;
      if constexpr (kBf16) {
        uint32_t hi, lo;
        split_bf16(p, hi, lo);
        p16_lds[wave][0][h][lane] = (uint16_t)hi;
        p16_lds[wave][1][h][lane] = (uint16_t)lo;
      } else
        p_lds[wave][h][lane] = p;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < DL; ++k) o[h][k] *= alpha[h];
    // The weights are private to this wave: a wavefront-scope fence orders the
    // LDS writes above before the broadcast reads below.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------- P*V: one lane per value dimension ----------------
#pragma unroll
    for (int c16 = 0; c16 < kTile; c16 += 16) {
      const int tok = tok0 + c16;
      if (tok >= end) break;
      const int pid = ptab[tok >> a.page_shift];
      if (pid < 0 || pid >= a.num_pages) continue;  // flagged in the score pass
      const int slot = tok & (P - 1);
      const int nvalid = min(16, end - tok);
      // Value runs of all the lane's dimensions first, then heads outer and
      // dimensions inner, so each head's weights are read from LDS once per run.
      uint32_t vw[DL][kBf16 ? 8 : 16];
#pragma unroll
      for (int k = 0; k < DL; ++k) {
        const int d = lane + 64 * k;
        const T* vp = static_cast<const T*>(a.v) + (((int64_t)pid * a.H_kv + t.kvh) * D + d) * P + slot;
#pragma unroll
        for (int q4 = 0; q4 < (kBf16 ? 2 : 4); ++q4) {
          const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp + q4 * (16 / sizeof(T))));
#pragma unroll
          for (int e = 0; e < 4; ++e) vw[k][4 * q4 + e] = x[e];
        }
        if (nvalid < 16) {   // zero values past `end` (poisoned or foreign slots)
          if constexpr (kBf16) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              vw[k][e] &= ((2 * e < nvalid) ? 0x0000FFFFu : 0u) | ((2 * e + 1 < nvalid) ? 0xFFFF0000u : 0u);
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) vw[k][e] = e < nvalid ? vw[k][e] : 0u;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if constexpr (kBf16) {
          const u32x4_t* ph = reinterpret_cast<const u32x4_t*>(&p16_lds[wave][0][h][c16]);
          const u32x4_t* pl = reinterpret_cast<const u32x4_t*>(&p16_lds[wave][1][h][c16]);
          const u32x4_t h0 = ph[0], h1 = ph[1], l0 = pl[0], l1 = pl[1];
          const uint32_t hw[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          const uint32_t lw[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
          for (int k = 0; k < DL; ++k) {
            float acc = o[h][k];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              acc = dot2_bf16(hw[e], vw[k][e], acc);
              acc = dot2_bf16(lw[e], vw[k][e], acc);
            }
            o[h][k] = acc;
          }
        } else {
          const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(&p_lds[wave][h][c16]);
          const f32x4_t p4[4] = {pp[0], pp[1], pp[2], pp[3]};
#pragma unroll
          for (int k = 0; k < DL; ++k) {
            float acc = o[h][k];
#pragma unroll
            for (int e = 0; e < 16; ++e) acc = fmaf(p4[e >> 2][e & 3], __uint_as_float(vw[k][e]), acc);
            o[h][k] = acc;
          }
        }
      }
    }
  }

  // ---------------- merge the four waves' states through LDS ----------------
  if (lane == 0) bad_lds[wave] = __builtin_amdgcn_ballot_w64(bad) != 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float ls = wave_sum(l[h]);
    if (lane == 0) {
      m_lds[wave][h] = m[h];
      l_lds[wave][h] = ls;
    }
#pragma unroll
    for (int k = 0; k < DL; ++k) o_lds[wave][h][lane + 64 * k] = o[h][k];
  }
  __syncthreads();
  if (bad_lds[0] | bad_lds[1] | bad_lds[2] | bad_lds[3]) {
    write_nan_state(a.o_part, a.lse_part, t.out_row, G, D);
    return;
  }
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_lds[w][h]);
    float Z = 0.f, acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = fast_exp2(m_lds[w][h] - M);
        Z += sc * l_lds[w][h];
        acc += sc * o_lds[w][h][d];
      }
    }
    const int64_t row = (int64_t)t.out_row + h;
    a.o_part[row * D + d] = M == -INFINITY ? 0.f : acc / Z;
    if (d == 0) a.lse_part[row] = M == -INFINITY ? -INFINITY : (M + fast_log2(Z)) * kLn2;
  }
}

// One work-group per task, in the plan's queue order.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void gqa_valu_kernel(ValuArgs a) {
  __shared__ ValuShared<T, D, G> sh;
  gqa_valu_task<T, D, G>(a, a.tasks[blockIdx.x], sh);
}

// Attention and merge in one launch (fused.hpp): the task, then the
// reduction role when every task has started.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void gqa_valu_fused(ValuArgs a, FusedArgs f) {
  __shared__ ValuShared<T, D, G> sh;
  __shared__ int slot;
  count_started(f);
  const DevTask t = a.tasks[blockIdx.x];
  gqa_valu_task<T, D, G>(a, t, sh);
  publish_task(f, t.b);
  if (all_started(f, &slot)) reduce_phase<D>(f, a.err_flag);
}

template <typename T, int D, int G>
static hipError_t launch_t(const AttnLaunch& L, const ValuArgs& args, const FusedLaunch* F) {
  if (F)
    hipLaunchKernelGGL((gqa_valu_fused<T, D, G>), dim3(L.num_tasks), dim3(256), 0, L.stream, args,
                       fused_args(*F));
  else
    hipLaunchKernelGGL((gqa_valu_kernel<T, D, G>), dim3(L.num_tasks), dim3(256), 0, L.stream, args);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_g(const AttnLaunch& L, const ValuArgs& args, int G, const FusedLaunch* F) {
  switch (G) {
    case 1: return launch_t<T, D, 1>(L, args, F);
    case 2: return launch_t<T, D, 2>(L, args, F);
    case 4: return launch_t<T, D, 4>(L, args, F);
    case 8: return launch_t<T, D, 8>(L, args, F);
    case 16: return launch_t<T, D, 16>(L, args, F);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_valu(const AttnLaunch& L, const FusedLaunch* F) {
  const skv_attn_desc& d = *L.desc;
  ValuArgs args;
  args.q = L.q;
  args.k = L.k_pages;
  args.v = L.v_pages;
  args.page_table = L.page_table;
  args.seq_lens = L.seq_lens;
  args.tasks = reinterpret_cast<const DevTask*>(static_cast<const uint8_t*>(L.workspace) + L.tasks_off);
  args.err_flag = reinterpret_cast<int32_t*>(const_cast<void*>(L.workspace));
  args.o_part = L.o_part;
  args.lse_part = L.lse_part;
  args.H_q = d.num_q_heads;
  args.H_kv = d.num_kv_heads;
  args.page_shift = __builtin_ctz((unsigned)d.page_size);
  args.max_pages = d.max_pages_per_seq;
  args.num_pages = d.num_pages;
  args.scale_log2 = d.softmax_scale * kLog2e;
  const int G = d.num_q_heads / d.num_kv_heads;
  if (L.num_tasks == 0) return hipSuccess;
  if (d.dtype == SKV_BF16) {
    if (d.head_dim_qk == 64) return launch_g<uint16_t, 64>(L, args, G, F);
    if (d.head_dim_qk == 128) return launch_g<uint16_t, 128>(L, args, G, F);
  } else {
    if (d.head_dim_qk == 64) return launch_g<float, 64>(L, args, G, F);
    if (d.head_dim_qk == 128) return launch_g<float, 128>(L, args, G, F);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gqa_valu(const AttnLaunch& L) { return launch_valu(L, nullptr); }

hipError_t launch_gqa_valu_fused(const AttnLaunch& L, const FusedLaunch& F) { return launch_valu(L, &F); }

}  // namespace skv
