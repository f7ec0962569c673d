// Paged split-KV partial attention for GQA groups of 16 (or 8) query heads per
// KV head (bf16 storage, fp32 accumulation) on the matrix cores.
//
// A group of 8 fills the 16 head columns of the products with copies of its
// heads (lane n takes head n mod 8) and writes 8 rows: the matrix cores stay a
// small share of the time (the kernel streams KV bytes), and the stream runs
// as fast as for 16 heads (8 heads on the vector-ALU kernel left it half
// bound by its dot products).
//
// One work-group (4 waves) runs one task: the 16 query heads of one KV head for
// one query token, over the KV range [lo, end) of one split. The waves take the
// split's 32-token steps round-robin; each keeps its own online-softmax state,
// and the four states are merged through LDS into the split's partial state
// (output normalised over the split plus natural-log LSE; LiquidCP section 2.1
// and Equation 1).
//
// Per 32-token step a wave issues two products with v_mfma_f32_16x16x32_bf16:
//   S^T[16 tokens x 16 heads]  = K[16 x D] * Q^T[D x 16]     (two token blocks)
//   O^T[16 dims  x 16 heads]  += V^T[16 x 32 tokens] * P^T[32 tokens x 16 heads]
// Every lane owns one head (lane % 16) in both outputs, so the softmax rescale
// needs no data movement, and the S^T output registers are exactly the P^T
// operand of the second product once packed to bf16 (as a hi + lo pair of bf16
// terms, two products per step). The storage layouts make
// every operand a direct, coalesced load from HBM into registers: keys as
// [D/8][P][8] per page (16 consecutive tokens of one 16-byte chunk are 256
// contiguous bytes), values dimension-major [D][P] per page (a lane's 4 tokens
// of one dimension are 8 contiguous bytes). No LDS is used until the final
// merge of the four waves.
//
// FP8 KV (OCP E4M3 codes with a float32 scale per page and KV head; SPLASH
// appendix C.1 serves an FP8 E4M3 KV cache): the same layouts at one byte per
// element, so a lane's key load is one 16-byte chunk of 16 dimensions (the
// operands of two consecutive products; the query operand takes the same
// dimension order). The step's tokens are ordered so that a lane's value load
// is 8 bytes (8 consecutive tokens of one dimension, within one page) rather
// than two 4-byte loads: the score rows of each product are taken in runs of
// 4 tokens (StepRegs8). v_cvt_scalef32_pk_bf16_fp8 turns two codes into two
// bf16 in one instruction, exactly (every E4M3 value is a bf16 value), and the
// products run as for bf16 storage. Each 16-token half of a step lies in one
// page (P >= 16) and a lane's tokens lie in one half, so the half's key scale
// multiplies the lane's scores and its value scale the lane's softmax weights
// before the P*V product (the normaliser sums the unscaled weights). The
// matrix cores' own FP8 products would need the queries and weights in FP8 as
// well, which costs far more accuracy than this stream has to spend time.
#include "device_common.hpp"
#include "fused.hpp"
#include "internal.hpp"

#ifndef RING_STEPS
#define RING_STEPS 4
#endif

namespace skv {

struct MfmaArgs {
  const uint16_t* q;
  const uint8_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const DevTask* tasks;
  int32_t* err_flag;
  float* o_part;
  float* lse_part;
  const float* k_scale;   // FP8 KV: [num_pages][H_kv]
  const float* v_scale;
  int32_t H_q, H_kv, G, page_shift, max_pages, num_pages;
  float scale_log2;
};

namespace {

constexpr int kG = 16;       // query heads per KV head
constexpr int kWaves = 4;
constexpr int kStep = 32;    // tokens per wave step (two 16-token MFMA blocks)

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
struct StepRegs {
  u32x4_t k[2][D / 32];   // A operand of S^T for token blocks 0 and 1
  u32x2_t v[2][D / 16];   // 4 tokens x 1 dimension per block, per 16-dim group
};

// Read-only inputs addressed through the constant address space: wave-uniform
// loads from it become scalar loads (lgkmcnt), so a page id or scale the wave
// waits for does not drain the vector loads already in flight (vmcnt counts
// in issue order).
typedef const __attribute__((address_space(4))) int32_t const_i32_t;
typedef const __attribute__((address_space(4))) float const_f32_t;

template <int D>
struct Ctx {
  const MfmaArgs* a;
  const_i32_t* ptab;
  int64_t kvh;
  int end;
  int lane, g, r16;  // g = lane / 16 (k-group), r16 = lane % 16
};

// Issue the loads of the 32-token step starting at t0 (t0 < end). Returns
// true if a page id of the step is outside the pool: that page is not read
// (zeros stand in for it) and the task's state is written as NaN.
template <int D>
__device__ __forceinline__ bool load_step(const Ctx<D>& c, int t0, StepRegs<D>& s) {
  const MfmaArgs& a = *c.a;
  const int P = 1 << a.page_shift;
  bool bad = false;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int tb = t0 + 16 * blk;
    int pid = -1;
    if (tb < c.end) {
      pid = c.ptab[tb >> a.page_shift];
      if (pid < 0 || pid >= a.num_pages) {
        if (c.lane == 0) raise_error(a.err_flag, kErrPageId);
        bad = true;
        pid = -1;
      }
    }
    if (pid >= 0) {
      const int slot = tb & (P - 1);
      const int64_t ph = (int64_t)pid * a.H_kv + c.kvh;   // page-head block
      const uint8_t* kp = a.k + (ph * (D / 8) * P + slot + c.r16) * 16;
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        s.k[blk][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + (int64_t)(4 * m + c.g) * P * 16));
      const uint16_t* vp = a.v + (ph * D + c.r16) * P + slot + 4 * c.g;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
        s.v[blk][nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vp + (int64_t)16 * nb * P));
    } else {
#pragma unroll
      for (int m = 0; m < D / 32; ++m) s.k[blk][m] = u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) s.v[blk][nb] = u32x2_t{0, 0};
    }
  }
  return bad;
}

// FP8 KV: one step's raw codes and the scales of its two 16-token halves
// (each half lies in one page). The step's tokens are ordered so that a lane
// holds 8 consecutive tokens of one dimension in the value operand (one 8-byte
// load): score block blk row r is token 8 (r / 4) + 4 blk + r % 4, so lane
// (g, r16) gets the scores of tokens 8 g + 4 blk + e, and the k-index 8 g + i
// of the P*V product is token 8 g + i.
template <int D>
struct StepRegs8 {
  u32x4_t k[2][D / 64];   // block blk: 16 codes (dims 16 (4j + g) .. + 15) of its row r16's token
  uint32_t v[2][D / 16];  // dimension 16 nb + r16: tokens 8g .. 8g + 3 (v[0]) and 8g + 4 .. + 7 (v[1])
  float ks[2], vs[2];     // per half
};

template <int D>
__device__ __forceinline__ bool load_step8(const Ctx<D>& c, int t0, StepRegs8<D>& s) {
  const MfmaArgs& a = *c.a;
  const int P = 1 << a.page_shift;
  bool bad = false;
  int64_t ph[2] = {0, 0};   // page-head block of each half
  int slot[2] = {0, 0};
  bool ok[2] = {false, false};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int th = t0 + 16 * h;
    s.ks[h] = 0.f;
    s.vs[h] = 0.f;
    if (th < c.end) {
      const int pid = c.ptab[th >> a.page_shift];
      if (pid < 0 || pid >= a.num_pages) {
        if (c.lane == 0) raise_error(a.err_flag, kErrPageId);
        bad = true;
      } else {
        ok[h] = true;
        slot[h] = th & (P - 1);
        ph[h] = (int64_t)pid * a.H_kv + c.kvh;
        s.ks[h] = ((const_f32_t*)a.k_scale)[ph[h]];
        s.vs[h] = ((const_f32_t*)a.v_scale)[ph[h]];
      }
    }
  }
  // keys: row r16 of block blk is token 8 (r16 / 4) + 4 blk + r16 % 4, in
  // half r16 / 8
  const int kh = c.r16 >> 3;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int tok = 8 * ((c.r16 >> 2) & 1) + 4 * blk + (c.r16 & 3);   // within the half
    const uint8_t* kp = a.k + ((kh ? ph[1] : ph[0]) * (D / 16) * P + (kh ? slot[1] : slot[0]) + tok) * 16;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      u32x4_t w = {0, 0, 0, 0};
      if (kh ? ok[1] : ok[0])
        w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + (int64_t)(4 * j + c.g) * P * 16));
      s.k[blk][j] = w;
    }
  }
  // values: tokens 8 (g % 2) .. + 7 of half g / 2, 8 bytes
  const int vh = c.g >> 1;
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.v) + ((vh ? ph[1] : ph[0]) * D + c.r16) * P +
                      (vh ? slot[1] : slot[0]) + 8 * (c.g & 1);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    u32x2_t w = {0u, 0u};
    if (vh ? ok[1] : ok[0]) w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vp + (int64_t)16 * nb * P));
    s.v[0][nb] = w[0];
    s.v[1][nb] = w[1];
  }
  return bad;
}

// Two E4M3 codes (byte pair kHi of w) as two bf16 in one word.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// Codes to the bf16 operand registers of compute_step (product 2j takes the
// low 8 codes of chunk j, product 2j + 1 the high 8).
template <int D>
__device__ __forceinline__ void decode_step(const StepRegs8<D>& r, StepRegs<D>& s) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const u32x4_t w = r.k[blk][j];
      s.k[blk][2 * j] = u32x4_t{e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
                                e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
      s.k[blk][2 * j + 1] = u32x4_t{e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
                                    e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
      s.v[blk][nb] = u32x2_t{e4m3x2_to_bf16x2<false>(r.v[blk][nb]), e4m3x2_to_bf16x2<true>(r.v[blk][nb])};
  }
}

template <int D>
struct State {
  float m, l;
  f32x4_t o[D / 16];
};

// kmul / vmul (FP8 KV): the factor of the lane's scores (softmax scale in
// log2 units times the key scale) and of its weights (value scale). With kF8
// the step's tokens take the FP8 order (StepRegs8): lane (g, r16)'s scores
// of block blk are tokens 8 g + 4 blk + e; otherwise 16 blk + 4 g + e.
template <int D, bool kF8 = false>
__device__ __forceinline__ void compute_step(const Ctx<D>& c, int t0, StepRegs<D>& s,
                                             const u32x4_t (&qf)[D / 32], State<D>& st,
                                             float scale_log2, const float* kmul = nullptr,
                                             const float* vmul = nullptr) {
  // scores S^T for both token blocks
  f32x4_t sc[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) acc = mfma16(s.k[blk][m], qf[m], acc);
    sc[blk] = acc;
  }
  // mask, scale to log2 units, row (= head) maximum over the 32 tokens
  const bool tail = t0 + kStep > c.end;
  float sv[8];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = t0 + (kF8 ? 8 * c.g + 4 * blk : 16 * blk + 4 * c.g) + e;
      const float x = sc[blk][e] * (kF8 ? *kmul : scale_log2);
      sv[4 * blk + e] = (!tail || tok < c.end) ? x : -INFINITY;
    }
  float mt = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
  mt = max_xor32(max_xor16(mt));
  const float mn = fmaxf(st.m, mt);
  const float alpha = fast_exp2(st.m - mn);
  // the accumulators need rescaling only where a head's maximum rose
  // (elsewhere alpha is exactly 1; at the first step they are zero)
  const bool rescale = __builtin_amdgcn_ballot_w64(mn != st.m) != 0;
  st.m = mn;
  float p[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = fast_exp2(sv[i] - mn);
    ps += p[i];
  }
  st.l = st.l * alpha + ps;
  // P^T operand as two bf16 terms (hi + lo): the second product costs matrix
  // throughput that this HBM-bound kernel has to spare, and keeps ~16 bits of
  // each weight instead of 8.
  uint32_t ph[4], pl[4];
  if constexpr (kF8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(p[2 * i] * *vmul, p[2 * i + 1] * *vmul, ph[i], pl[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(p[2 * i], p[2 * i + 1], ph[i], pl[i]);
  }
  const u32x4_t pf_hi = {ph[0], ph[1], ph[2], ph[3]};
  const u32x4_t pf_lo = {pl[0], pl[1], pl[2], pl[3]};
  // values past `end` (the split's end, or poisoned slots of the last page)
  // are zeroed so that 0 * NaN cannot reach the accumulator
  if (tail) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int tok = t0 + (kF8 ? 8 * c.g + 4 * blk : 16 * blk + 4 * c.g);
      const int nv = c.end - tok;  // valid tokens among this lane's 4
      if (nv < 4) {
        const uint32_t m0 = nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0x0000FFFFu : 0u);
        const uint32_t m1 = nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0x0000FFFFu : 0u);
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          s.v[blk][nb][0] &= m0;
          s.v[blk][nb][1] &= m1;
        }
      }
    }
  }
  if (rescale) {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[nb] *= alpha;
  }
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const u32x4_t vf = {s.v[0][nb][0], s.v[0][nb][1], s.v[1][nb][0], s.v[1][nb][1]};
    st.o[nb] = mfma16(vf, pf_hi, st.o[nb]);
    st.o[nb] = mfma16(vf, pf_lo, st.o[nb]);
  }
}

// LDS of one work-group: the four waves' states for the final merge.
template <int D>
struct MfmaShared {
  float m_lds[kWaves][kG], l_lds[kWaves][kG];
  float o_lds[kWaves][kG][D + 4];
  int bad_lds[kWaves];
};

// One task: the query heads of one KV head for one query token over the KV
// range [lo, end) of one split, written as the split's partial state.
template <int D, bool kF8 = false>
__device__ __forceinline__ void gqa_mfma_task(const MfmaArgs& a, const DevTask& t, MfmaShared<D>& sh) {
  auto& m_lds = sh.m_lds;
  auto& l_lds = sh.l_lds;
  auto& o_lds = sh.o_lds;
  auto& bad_lds = sh.bad_lds;
  if (a.seq_lens[t.b] != t.seq_len) {
    // the device lengths are not the ones the plan was built from: no KV is
    // read and the state is NaN (uniform over the work-group: one task)
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrSeqLen);
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.G, D);
    return;
  }
  Ctx<D> c;
  c.a = &a;
  c.lane = threadIdx.x & 63;
  c.g = c.lane >> 4;
  c.r16 = c.lane & 15;
  c.kvh = t.kvh;
  c.end = t.end;
  c.ptab = (const_i32_t*)(a.page_table + (int64_t)t.b * a.max_pages);
  // wave-uniform (readfirstlane): the step positions, page ids and scales
  // derived from it stay scalar, so page ids come by scalar loads and waiting
  // for one does not drain the vector loads already in flight
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Q^T operand: lane owns head r16; its k-slots of product m are dims
  // 8(4m+g)..+7 (FP8 KV: 16(4(m/2)+g) + 8(m%2)..+7, the key chunk order)
  u32x4_t qf[D / 32];
  {
    // groups of G < 16 heads: lanes past G compute copies of the group's heads
    const uint16_t* qp = a.q + ((int64_t)t.q_row * a.H_q + (int64_t)t.kvh * a.G + (c.r16 & (a.G - 1))) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const int dim0 = kF8 ? 16 * (4 * (m >> 1) + c.g) + 8 * (m & 1) : 8 * (4 * m + c.g);
      qf[m] = *reinterpret_cast<const u32x4_t*>(qp + dim0);
    }
  }

  State<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) st.o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Two register sets alternate so that one step's loads are in flight while
  // the previous step is computed.
  constexpr int kStride = kWaves * kStep;
  int t0 = t.lo + wave * kStep;
  bool bad = false;   // wave-uniform: the page ids are per 16-token block
  if constexpr (kF8) {
    // a ring of kRing raw steps: loads run kRing - 1 steps ahead (a step of
    // codes is half a bf16 step's bytes, so more of them stay in flight)
    constexpr int kRing = 3;
    StepRegs8<D> r[kRing];
    StepRegs<D> s;
    // one step's codes decoded, with its blocks' score and weight factors
    auto step = [&](int ts, const StepRegs8<D>& rr) {
      decode_step(rr, s);
      // the lane's tokens all lie in half g / 2
      const float km = a.scale_log2 * (c.g >> 1 ? rr.ks[1] : rr.ks[0]);
      const float vm = c.g >> 1 ? rr.vs[1] : rr.vs[0];
      compute_step<D, true>(c, ts, s, qf, st, a.scale_log2, &km, &vm);
    };
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i)
      if (t0 + i * kStride < c.end) bad |= load_step8(c, t0 + i * kStride, r[i]);
    while (t0 < c.end) {
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        const int tl = t0 + (kRing - 1) * kStride;
        if (tl < c.end) bad |= load_step8(c, tl, r[(i + kRing - 1) % kRing]);
        step(t0, r[i]);
        t0 += kStride;
        if (t0 >= c.end) break;
      }
    }
  } else {
    StepRegs<D> ra, rb;
    if (t0 < c.end) bad |= load_step(c, t0, ra);
    while (t0 < c.end) {
      const int t1 = t0 + kStride;
      if (t1 < c.end) bad |= load_step(c, t1, rb);
      compute_step(c, t0, ra, qf, st, a.scale_log2);
      if (t1 >= c.end) break;
      const int t2 = t1 + kStride;
      if (t2 < c.end) bad |= load_step(c, t2, ra);
      compute_step(c, t1, rb, qf, st, a.scale_log2);
      t0 = t2;
    }
  }

  // Merge the four waves' states: sum l over the 4 lanes of each head first.
  float l = st.l;
  l = sum_xor32(sum_xor16(l));
  if (c.g == 0) {
    m_lds[wave][c.r16] = st.m;
    l_lds[wave][c.r16] = l;
  }
  if (c.lane == 0) bad_lds[wave] = bad;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) o_lds[wave][c.r16][16 * nb + 4 * c.g + e] = st.o[nb][e];
  __syncthreads();
  if (bad_lds[0] | bad_lds[1] | bad_lds[2] | bad_lds[3]) {
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.G, D);
    return;
  }
  for (int i = threadIdx.x; i < a.G * D; i += 256) {
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

// ---------------------------------------------------------------------------
// Tasks of several query tokens (a query tile of one request: up to
// kTileRows / G consecutive tokens). The rows (row = token * G + head) are
// columns of the products in blocks of 16; wave w owns blocks 2w and 2w + 1
// (rows 32w .. 32w + 31) for the whole split, so a wave's state needs no
// merge with the others'. The split's keys and values pass through LDS once
// per work-group: each 32-token step is copied by the LDS DMA
// (global_load_lds_dwordx4: lane i's 16 bytes land at the instruction's LDS
// base + 16 i) into a ring of kRing steps, issued kRing - 1 steps ahead of
// its use, and every wave reads its operands from there, each key and value
// fragment once for both of its blocks. Step layout in LDS:
//   keys   [D/8 chunks][32 tokens][16 bytes]: the page's own chunk-major order,
//          so a 16-lane read of one chunk is 256 contiguous bytes; the lanes
//          a 16-byte read serves together (8 of one 16-lane group with the
//          other half of the neighbouring group) then read tokens 0-7 of one
//          chunk and 8-15 of the next, different banks;
//   values [D dims][32 tokens] (64 bytes per dimension) in 8-byte slots of 4
//          tokens, slot (token / 4) ^ (2 ((dim / 4) % 4)): the 32 lanes one
//          8-byte read serves (16 dimensions x two token groups) then cover
//          all 64 banks. A 16-byte DMA chunk (8 tokens of one dimension) keeps
//          its two slots adjacent, the XOR being even. The reads stay single
//          8-byte reads: paired into two-address reads (ds_read2_b64, which
//          the compiler forms from reads a fixed distance apart) they measured
//          8 bank-conflict cycles each with the bank-conflict counter, single
//          reads and the key reads none.
// Causal rows see their own end: lane n's column is one row, masked at
// min(split end, the visible end of its token).
// ---------------------------------------------------------------------------

constexpr int kTileRows = 128;  // rows of a full query tile
constexpr int kRing = RING_STEPS;        // LDS steps in the ring
constexpr int kRowsBPW = 2;     // column blocks per wave

constexpr int kVGroupBytes = 1024;                // 16 dimensions of values
template <int D>
constexpr int kKeyBytes = kStep * D * 2;          // keys of one step
template <int D>
constexpr int kStepBytes = kKeyBytes<D> + (D / 16) * kVGroupBytes;
template <int D>
constexpr int kStepBlocks = 2 * kKeyBytes<D> / 1024;   // 1 KB DMA blocks per step (keys, then values)
template <int D>
constexpr int kDmaPerWaveStep = kStepBlocks<D> / kWaves;

template <int D>
struct RowsShared {
  __attribute__((aligned(16))) uint8_t ring[kRing][kStepBytes<D>];
};

// The rows of a multi-token task written as NaN (a device error).
template <int D>
__device__ __forceinline__ void rows_nan(const MfmaArgs& a, const DevTask& t) {
  for (int j = 0; j < t.ntok; ++j)
    write_nan_state(a.o_part, a.lse_part, (int64_t)t.out_row + (int64_t)j * a.H_q, a.G, D);
}

typedef __attribute__((address_space(3))) void rows_lds_void_t;

// One DMA instruction: each lane's 16 bytes at `src` to LDS byte
// lds + 16 lane (M0 carries the LDS base; one wait state separates its write
// from the DMA). Inline assembly, so that the compiler does not track these
// loads: the loop orders them with its own vmcnt waits (the vector-memory
// counter retires in order).
__device__ __forceinline__ void rows_dma(const uint8_t* src, uint32_t lds) {
  __asm__ __volatile__("s_mov_b32 m0, %[l]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[p], off nt"
                       :
                       : [l] "s"(lds), [p] "v"(src)
                       : "memory", "m0");
}

// s_waitcnt immediates for the vector-memory counter only (gfx9 encoding).
template <int N>
constexpr int kRowsWaitVm = 0x3f70 | (N & 15) | ((N >> 4) << 14);

// Wait until at most `ahead` steps of this wave's DMAs are in flight.
template <int D, int N = kRing - 2>
__device__ __forceinline__ void rows_wait_ahead(int ahead) {
  if constexpr (N == 0) {
    __builtin_amdgcn_s_waitcnt(kRowsWaitVm<0>);
  } else {
    if (ahead >= N) __builtin_amdgcn_s_waitcnt(kRowsWaitVm<N * kDmaPerWaveStep<D>>);
    else rows_wait_ahead<D, N - 1>(ahead);
  }
}

__device__ __forceinline__ void rows_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Page ids of the step at t0 (its two 16-token halves), wave-uniform scalars
// read one step before they are used, so the scalar-load latency is not paid
// at every step. Indices past the request's last page are clamped to it (those
// tokens are masked where they are used).
struct StepPages {
  int p0, p1;
};
__device__ __forceinline__ StepPages step_pages(const MfmaArgs& a, const_i32_t* ptab, int t0, int end) {
  const int last = (end - 1) >> a.page_shift;
  return StepPages{ptab[min(t0 >> a.page_shift, last)], ptab[min((t0 + 16) >> a.page_shift, last)]};
}

// This wave's DMA blocks of a step (kDmaPerWaveStep<D> blocks: wave, wave +
// 4, ...; a block below kStepBlocks / 2 holds keys, the rest values). Each
// lane's source is a per-step base of the page half it reads (keys: the
// lane's token, values: its 4-token group) plus a lane offset fixed for the
// task plus a per-block step, so a step costs a few scalar operations and one
// select and 64-bit add per block. An id outside the pool is never
// dereferenced: page 0 stands in and the task's state is written as NaN.
template <int D>
struct RowsDma {
  static constexpr int kHalf = kDmaPerWaveStep<D> / 2;   // key blocks per wave
  uint32_t koff, voff;    // lane offsets (bytes) from the half's base
  bool khi, vhi;          // the lane's token lies in the step's second half
  uint32_t ldsoff[kDmaPerWaveStep<D>];   // wave-uniform LDS offsets within a step

  // once per task
  __device__ __forceinline__ void setup(const MfmaArgs& a, int wave, int lane) {
    const int P = 1 << a.page_shift;
    // keys: block wave + 4 j holds chunks 2 blk, 2 blk + 1 of the 32 tokens
    // (slot 64 blk + lane: chunk (64 blk + lane) / 32, token lane % 32)
    const int tk = lane & 31;
    khi = tk >= 16;
    const int tkp = P >= 32 ? tk : (tk & 15);           // token within its page row run
    koff = (uint32_t)(((2 * wave + (lane >> 5)) * P + tkp) * 16);
    // values: block kStepBlocks / 2 + wave + 4 jv holds dims 16 (wave + 4 jv)
    // .. + 15; lane (d, pair): dimension lane / 4 of the block, the 4 tokens of
    // its 8-byte slot
    const int d = lane >> 2, pair = lane & 3;
    const int tv = 4 * ((2 * pair) ^ (2 * ((d >> 2) & 3)));
    vhi = tv >= 16;
    const int tvp = P >= 32 ? tv : (tv & 15);
    voff = (uint32_t)(((16 * wave + d) * P + tvp) * 2);
#pragma unroll
    for (int j = 0; j < kDmaPerWaveStep<D>; ++j) {
      const int blk = wave + kWaves * j;
      ldsoff[j] = j < kHalf ? 1024u * blk : (uint32_t)(kKeyBytes<D> + (blk - kStepBlocks<D> / 2) * kVGroupBytes);
    }
  }
  // Issue the step at t0 into the LDS step buffer lds_step; returns true if
  // a page id of the step is outside the pool.
  __device__ __forceinline__ bool issue(const MfmaArgs& a, StepPages pg, int kvh, int t0, uint32_t lds_step) const {
    const int P = 1 << a.page_shift;
    int p0 = pg.p0, p1 = pg.p1;
    const bool ok0 = p0 >= 0 && p0 < a.num_pages, ok1 = p1 >= 0 && p1 < a.num_pages;
    if (!ok0) p0 = 0;
    if (!ok1) p1 = 0;
    const int64_t ph0 = (int64_t)p0 * a.H_kv + kvh, ph1 = (int64_t)p1 * a.H_kv + kvh;
    // the step's first slot in its page (steps start at multiples of 32
    // tokens, splits at multiples of the 64-token KV tile: with P >= 32 the
    // step lies in one page, with P = 16 its halves are whole pages)
    const int64_t sl = P >= 32 ? (t0 & (P - 1)) : 0;
    const uint8_t* kb0 = a.k + (ph0 * (D / 8) * P + sl) * 16;
    const uint8_t* kb1 = a.k + (ph1 * (D / 8) * P + sl) * 16;
    const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(a.v) + (ph0 * D * P + sl) * 2;
    const uint8_t* vb1 = reinterpret_cast<const uint8_t*>(a.v) + (ph1 * D * P + sl) * 2;
    const uint8_t* kb = (khi ? kb1 : kb0) + koff;
    const uint8_t* vb = (vhi ? vb1 : vb0) + voff;
#pragma unroll
    for (int j = 0; j < kDmaPerWaveStep<D>; ++j) {
      // key block j: chunks 8 j further (4 blocks of 2 chunks); value block
      // j - kHalf: 64 dimensions further
      const uint8_t* src = j < kHalf ? kb + (int64_t)(8 * j) * P * 16 : vb + (int64_t)(64 * (j - kHalf)) * P * 2;
      rows_dma(src, lds_step + ldsoff[j]);
    }
    return !ok0 || !ok1;
  }
};

template <int D>
__device__ __forceinline__ void gqa_rows_task(const MfmaArgs& a, const DevTask& task, RowsShared<D>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  DevTask t = task;
  t.b = __builtin_amdgcn_readfirstlane(task.b);
  t.kvh = __builtin_amdgcn_readfirstlane(task.kvh);
  t.lo = __builtin_amdgcn_readfirstlane(task.lo);
  t.end = __builtin_amdgcn_readfirstlane(task.end);
  t.q_row = __builtin_amdgcn_readfirstlane(task.q_row);
  t.out_row = __builtin_amdgcn_readfirstlane(task.out_row);
  t.ntok = __builtin_amdgcn_readfirstlane(task.ntok);
  t.hi = __builtin_amdgcn_readfirstlane(task.hi);
  t.vis_last = __builtin_amdgcn_readfirstlane(task.vis_last);
  t.step = __builtin_amdgcn_readfirstlane(task.step);
  if (a.seq_lens[t.b] != task.seq_len) {
    // the device lengths are not the ones the plan was built from: no KV is
    // read and the state is NaN (uniform over the work-group: one task)
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrSeqLen);
    rows_nan<D>(a, t);
    return;
  }
  const int G = a.G;
  const int R = G * t.ntok;                       // rows of the task
  const int CB = (R + 15) >> 4;                   // column blocks in use
  const int nblk = max(0, min(kRowsBPW, CB - kRowsBPW * wave));   // this wave's (uniform)
  const int end = t.end;
  const_i32_t* ptab = (const_i32_t*)(a.page_table + (int64_t)t.b * a.max_pages);

  // Q^T operands and per-column visible ends of the wave's blocks (rows past
  // the task's last are computed on a copy of the last row, not written)
  u32x4_t qf[kRowsBPW][D / 32];
  int end_col[kRowsBPW];
#pragma unroll
  for (int j = 0; j < kRowsBPW; ++j) {
    const int r = min(16 * (kRowsBPW * wave + j) + r16, R - 1);
    const int tok = r / G, h = r - tok * G;
    const uint16_t* qp = a.q + ((int64_t)(t.q_row + tok) * a.H_q + (int64_t)t.kvh * G + h) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) qf[j][m] = *reinterpret_cast<const u32x4_t*>(qp + 8 * (4 * m + g));
    end_col[j] = min(t.hi, t.vis_last - (t.ntok - 1 - tok) * t.step);
  }
  // the least visible end among the wave's columns (that of its first row's
  // token: a column's end grows with its token): steps wholly before it need
  // no mask
  const int end_min = __builtin_amdgcn_readfirstlane(
      min(t.hi, t.vis_last - (t.ntok - 1 - min(16 * kRowsBPW * wave, R - 1) / G) * t.step));
  // Q has landed before the first DMA (otherwise the compiler's wait for it
  // would sit inside the loop and drain the ring)
  __builtin_amdgcn_s_waitcnt(kRowsWaitVm<0>);

  float mrow[kRowsBPW], lrow[kRowsBPW];
  f32x4_t o[kRowsBPW][D / 16];
#pragma unroll
  for (int j = 0; j < kRowsBPW; ++j) {
    mrow[j] = -INFINITY;
    lrow[j] = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) o[j][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(rows_lds_void_t*)&sh.ring[0][0]);
  // per-lane LDS byte offsets of the operand reads within a step
  uint32_t koff[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) koff[blk] = (uint32_t)((g * 32 + 16 * blk + r16) * 16);
  uint32_t voff[2][D / 16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const int d = 16 * nb + r16, tg = 4 * blk + g;
      voff[blk][nb] = (uint32_t)(kKeyBytes<D> + nb * kVGroupBytes + r16 * 64 + ((tg ^ (2 * ((d >> 2) & 3))) * 8));
      // opaque to the compiler, so that it does not pair two of these reads
      __asm__ __volatile__("" : "+v"(voff[blk][nb]));
    }

  const int nsteps = end > t.lo ? (end - t.lo + kStep - 1) / kStep : 0;
  bool bad = false;
  RowsDma<D> dm;
  dm.setup(a, wave, lane);
  StepPages pg{0, 0};   // page ids of the next step to send
  if (nsteps > 0) pg = step_pages(a, ptab, t.lo, end);
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) {
    if (i < nsteps) {
      bad |= dm.issue(a, pg, t.kvh, t.lo + i * kStep, ring_lds + (uint32_t)(i * kStepBytes<D>));
      pg = step_pages(a, ptab, t.lo + (i + 1) * kStep, end);   // clamped: always a valid entry
    }
  }
  // the loop runs the ring's buffers in order, unrolled once around the ring
  // so that every buffer offset is a constant of the LDS instructions
  for (int k0 = 0; k0 < nsteps; k0 += kRing)
#pragma unroll
  for (int u = 0; u < kRing; ++u) {
    const int k = k0 + u;
    if (k >= nsteps) break;
    // step k has landed for this wave (its DMAs retire in order), then for all
    rows_wait_ahead<D>(min(kRing - 2, nsteps - 1 - k));
    rows_barrier();
    // the DMA of step k + kRing - 1, into the buffer step k - 1 left (every
    // wave has passed this barrier, so its reads of that step are done)
    if (k + kRing - 1 < nsteps) {
      bad |= dm.issue(a, pg, t.kvh, t.lo + (k + kRing - 1) * kStep,
                      ring_lds + (uint32_t)(((u + kRing - 1) % kRing) * kStepBytes<D>));
      pg = step_pages(a, ptab, t.lo + (k + kRing) * kStep, end);
    }
    if (nblk == 0) continue;   // wave-uniform: this wave's rows are past the task's
    const uint8_t* st = sh.ring[u];
    const int t0 = t.lo + k * kStep;
    // key fragments of both token blocks and value fragments
    u32x4_t kf[2][D / 32];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        kf[blk][m] = *reinterpret_cast<const u32x4_t*>(st + koff[blk] + 4 * 32 * 16 * m);
    u32x2_t vf[2][D / 16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) vf[blk][nb] = *reinterpret_cast<const u32x2_t*>(st + voff[blk][nb]);
    // values past `end` hold stale or poisoned page data: zero them, so that
    // 0 * NaN cannot reach the accumulators
    if (t0 + kStep > end) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int nv = end - (t0 + 16 * blk + 4 * g);   // valid tokens among the lane's 4
        if (nv < 4) {
          const uint32_t m0 = nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0x0000FFFFu : 0u);
          const uint32_t m1 = nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0x0000FFFFu : 0u);
#pragma unroll
          for (int nb = 0; nb < D / 16; ++nb) {
            vf[blk][nb][0] &= m0;
            vf[blk][nb][1] &= m1;
          }
        }
      }
    }
    // both blocks always (a block past the task's rows computes on copies of
    // its last row and is not written): one straight-line body, in which the
    // compiler can overlap one block's softmax with the other's products
#pragma unroll
    for (int j = 0; j < kRowsBPW; ++j) {
      f32x4_t sc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < D / 32; ++m) acc = mfma16(kf[blk][m], qf[j][m], acc);
        sc[blk] = acc;
      }
      float sv[8];
      if (t0 + kStep > end_min) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = t0 + 16 * blk + 4 * g + e;
            sv[4 * blk + e] = tok < end_col[j] ? sc[blk][e] * a.scale_log2 : -INFINITY;
          }
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * blk + e] = sc[blk][e] * a.scale_log2;
      }
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
      mt = max_xor32(max_xor16(mt));
      const float mn = fmaxf(mrow[j], mt);
      // a column may see no key yet (its end precedes this step): keep a
      // finite reference so that its weights are exp2(-inf) = 0, not NaN
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(mrow[j] - mref);
      // the accumulators need rescaling only where a column's maximum rose
      // (elsewhere alpha is exactly 1, or the column has no weight yet and
      // its accumulators are zero): usually no column after the first steps
      const bool rescale = __builtin_amdgcn_ballot_w64(mn != mrow[j]) != 0;
      mrow[j] = mn;
      float p[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(sv[i] - mref);
        ps += p[i];
      }
      lrow[j] = lrow[j] * alpha + ps;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_bf16x2(p[2 * i], p[2 * i + 1], ph[i], pl[i]);
      const u32x4_t pf_hi = {ph[0], ph[1], ph[2], ph[3]};
      const u32x4_t pf_lo = {pl[0], pl[1], pl[2], pl[3]};
      if (rescale) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) o[j][nb] *= alpha;
      }
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const u32x4_t vv = {vf[0][nb][0], vf[0][nb][1], vf[1][nb][0], vf[1][nb][1]};
        o[j][nb] = mfma16(vv, pf_hi, o[j][nb]);
        o[j][nb] = mfma16(vv, pf_lo, o[j][nb]);
      }
    }
  }
  // every wave's DMAs have landed before the work-group leaves its LDS
  __builtin_amdgcn_s_waitcnt(kRowsWaitVm<0>);
  // a bad page id is seen by every wave that prepared a DMA of it; any wave
  // that saw one makes the whole task NaN
  const bool any_bad = __syncthreads_or(bad);
  if (any_bad) {
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrPageId);
    rows_nan<D>(a, t);
    return;
  }
#pragma unroll
  for (int j = 0; j < kRowsBPW; ++j) {
    if (j >= nblk) break;
    const int r = 16 * (kRowsBPW * wave + j) + r16;
    const float l = sum_xor32(sum_xor16(lrow[j]));
    if (r >= R) continue;
    const int tok = r / G, h = r - tok * G;
    const int64_t row = (int64_t)t.out_row + (int64_t)tok * a.H_q + h;
    const bool empty = mrow[j] == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
      *reinterpret_cast<f32x4_t*>(a.o_part + row * D + 16 * nb + 4 * g) = o[j][nb] * inv;
    if (g == 0) a.lse_part[row] = empty ? -INFINITY : (mrow[j] + fast_log2(l)) * kLn2;
  }
}

// Multi-token tasks: one work-group per task, in the plan's queue order.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gqa_rows_kernel(MfmaArgs a) {
  __shared__ RowsShared<D> sh;
  gqa_rows_task<D>(a, a.tasks[blockIdx.x], sh);
}

// Multi-token tasks with the merge in the same launch (fused.hpp).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gqa_rows_fused(MfmaArgs a, FusedArgs f) {
  __shared__ RowsShared<D> sh;
  __shared__ int slot;
  count_started(f);
  const DevTask t = a.tasks[blockIdx.x];
  gqa_rows_task<D>(a, t, sh);
  publish_task(f, t.b);
  if (all_started(f, &slot)) reduce_phase<D>(f, a.err_flag);
}

// One work-group per task, in the plan's queue order.
template <int D, bool kF8 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gqa_mfma_kernel(MfmaArgs a) {
  __shared__ MfmaShared<D> sh;
  gqa_mfma_task<D, kF8>(a, a.tasks[blockIdx.x], sh);
}

// Attention and merge in one launch (fused.hpp): the task, then the
// reduction role when every task has started.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gqa_mfma_fused(MfmaArgs a, FusedArgs f) {
  __shared__ MfmaShared<D> sh;
  __shared__ int slot;
  count_started(f);
  const DevTask t = a.tasks[blockIdx.x];
  gqa_mfma_task<D>(a, t, sh);
  publish_task(f, t.b);
  if (all_started(f, &slot)) reduce_phase<D>(f, a.err_flag);
}

}  // namespace

static MfmaArgs mfma_args(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  MfmaArgs a;
  a.q = static_cast<const uint16_t*>(L.q);
  a.k = static_cast<const uint8_t*>(L.k_pages);
  a.v = static_cast<const uint16_t*>(L.v_pages);
  a.page_table = L.page_table;
  a.seq_lens = L.seq_lens;
  a.tasks = reinterpret_cast<const DevTask*>(static_cast<const uint8_t*>(L.workspace) + L.tasks_off);
  a.err_flag = reinterpret_cast<int32_t*>(const_cast<void*>(L.workspace));
  a.o_part = L.o_part;
  a.lse_part = L.lse_part;
  a.k_scale = L.k_scales;
  a.v_scale = L.v_scales;
  a.H_q = d.num_q_heads;
  a.H_kv = d.num_kv_heads;
  a.G = d.num_q_heads / d.num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)d.page_size);
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.scale_log2 = d.softmax_scale * kLog2e;
  return a;
}

static bool mfma_supported(const skv_attn_desc& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (G == kG || G == kG / 2) && d.dtype == SKV_BF16 && (d.head_dim_qk == 128 || d.head_dim_qk == 64);
}

static bool fp8_supported(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  const int G = d.num_q_heads / d.num_kv_heads;
  return (G == kG || G == kG / 2) && d.dtype == SKV_FP8_E4M3 && (d.head_dim_qk == 128 || d.head_dim_qk == 64) &&
         L.max_ntok == 1 && L.k_scales && L.v_scales;
}

hipError_t launch_gqa_mfma(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  if (d.dtype == SKV_FP8_E4M3) {
    if (!fp8_supported(L)) return hipErrorInvalidValue;
    if (L.num_tasks == 0) return hipSuccess;
    const MfmaArgs a = mfma_args(L);
    if (d.head_dim_qk == 128)
      hipLaunchKernelGGL((gqa_mfma_kernel<128, true>), dim3(L.num_tasks), dim3(256), 0, L.stream, a);
    else
      hipLaunchKernelGGL((gqa_mfma_kernel<64, true>), dim3(L.num_tasks), dim3(256), 0, L.stream, a);
    return hipGetLastError();
  }
  if (!mfma_supported(d)) return hipErrorInvalidValue;
  if (L.num_tasks == 0) return hipSuccess;
  const MfmaArgs a = mfma_args(L);
  // plans with several query tokens per task run on the multi-token kernel
  if (L.max_ntok > 1 && L.max_ntok * a.G > kTileRows)
    return hipErrorInvalidValue;
  if (d.head_dim_qk == 128) {
    if (L.max_ntok > 1) hipLaunchKernelGGL(gqa_rows_kernel<128>, dim3(L.num_tasks), dim3(256), 0, L.stream, a);
    else hipLaunchKernelGGL(gqa_mfma_kernel<128>, dim3(L.num_tasks), dim3(256), 0, L.stream, a);
  } else {
    if (L.max_ntok > 1) hipLaunchKernelGGL(gqa_rows_kernel<64>, dim3(L.num_tasks), dim3(256), 0, L.stream, a);
    else hipLaunchKernelGGL(gqa_mfma_kernel<64>, dim3(L.num_tasks), dim3(256), 0, L.stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_gqa_mfma_fused(const AttnLaunch& L, const FusedLaunch& F) {
  const skv_attn_desc& d = *L.desc;
  if (!mfma_supported(d)) return hipErrorInvalidValue;
  const MfmaArgs a = mfma_args(L);
  const FusedArgs f = fused_args(F);
  if (L.max_ntok > 1 && L.max_ntok * a.G > kTileRows)
    return hipErrorInvalidValue;
  if (d.head_dim_qk == 128) {
    if (L.max_ntok > 1) hipLaunchKernelGGL(gqa_rows_fused<128>, dim3(L.num_tasks), dim3(256), 0, L.stream, a, f);
    else hipLaunchKernelGGL(gqa_mfma_fused<128>, dim3(L.num_tasks), dim3(256), 0, L.stream, a, f);
  } else {
    if (L.max_ntok > 1) hipLaunchKernelGGL(gqa_rows_fused<64>, dim3(L.num_tasks), dim3(256), 0, L.stream, a, f);
    else hipLaunchKernelGGL(gqa_mfma_fused<64>, dim3(L.num_tasks), dim3(256), 0, L.stream, a, f);
  }
  return hipGetLastError();
}

}  // namespace skv
