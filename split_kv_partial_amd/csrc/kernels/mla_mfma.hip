// Paged split-KV partial attention for absorbed multi-head latent attention
// (bf16, up to 128 query heads sharing one 576-wide latent row per token whose
// first 512 entries are the value), on the matrix cores.
//
// Shapes follow SPLASH sections 2-3: KV bytes per token L(d_c + d_r)b with
// d_c = 512 and d_r = 64; the attention at a request's owner computes rows
// [N_r, H, d_c + d_r] and returns width d_c. One work-group (8 waves) runs one
// task: all heads of one query token over the KV range [lo, end) of one split,
// so each latent row is read from HBM once per task and shared by every head
// (the reason MLA decode is matrix-core work: ~242 flop per KV byte).
//
// Work split inside the work-group: wave w owns head group hg = w / 2 (32 heads)
// and dimension half dh = w % 2. For a 32-token tile staged in LDS:
//   S^T[32 tok x 32 heads] partial over its 288 of the 576 qk dims
//       (v_mfma_f32_16x16x32_bf16; two token blocks x two 16-head blocks),
//   the two halves of a head group add their partial scores through LDS, so
//   both hold identical full scores and softmax state,
//   O^T[256 dims x 32 heads] += V^T[256 x 32 tok] * P^T[32 tok x 32 heads]
//       over its 256 of the 512 value dims.
// Every output element has exactly one owner wave, so no merge between waves
// is needed at the end. The V^T operand comes from the row-major latent tile
// through the gfx950 transposing LDS read (ds_read_b64_tr_b16: within each 16
// lanes, lane i addresses row i/4, columns 4(i%4)..+3 of a 4 x 16 block and lane
// n receives column n of its four rows), so the tile is stored in LDS once.
// Tiles are double-buffered in LDS; the next tile is fetched into registers
// while the current one is computed. Softmax weights enter P*V as one bf16
// term (max |error| <= 2^-9 |V|, within the bf16 tolerance for latent values).
#include "device_common.hpp"
#include "internal.hpp"

namespace skv {

struct MlaArgs {
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const DevTask* tasks;
  int32_t* err_flag;
  float* o_part;
  float* lse_part;
  int32_t H_q, page_shift, max_pages, num_pages;
  float scale_log2;
};

namespace {

constexpr int kD = 576;          // qk width: 512 latent + 64 rope
constexpr int kDv = 512;         // value width (the latent)
constexpr int kT = 32;           // tokens per tile
constexpr int kRS = kD + 8;      // LDS row stride in bf16 (16-byte pad)
constexpr int kChunks = kD / 8;  // 16-byte chunks per row (72)
constexpr int kThreads = 512;
constexpr int kStage = (kT * kChunks + kThreads - 1) / kThreads;  // chunks per thread (5)
constexpr int kKs = kD / 2 / 32;  // 32-wide k-steps per dimension half (9)
constexpr int kNb = kDv / 2 / 16; // 16-dim output blocks per dimension half (16)

typedef short __attribute__((__vector_size__(4 * sizeof(short)))) s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2_t tr_read(const uint16_t* lds_ptr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_ptr));
  return __builtin_bit_cast(u32x2_t, v);
}

struct Stage {
  u32x4_t r[kStage];
};

// Fetch the 32 x 576 tile at token t0 into registers (zeros past `end`).
__device__ __forceinline__ void fetch(const MlaArgs& a, const int32_t* ptab, int end, int t0,
                                      Stage& st) {
  const int P = 1 << a.page_shift;
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int c = threadIdx.x + kThreads * j;
    u32x4_t v = {0, 0, 0, 0};
    if (c < kT * kChunks) {
      const int tok = t0 + c / kChunks;
      if (tok < end) {
        const int pid = ptab[tok >> a.page_shift];
        if (pid >= 0 && pid < a.num_pages) {
          v = *reinterpret_cast<const u32x4_t*>(
              a.kv + (((int64_t)pid * P + (tok & (P - 1))) * kD + (c % kChunks) * 8) * 2);
        } else {
          raise_error(a.err_flag, 1);
        }
      }
    }
    st.r[j] = v;
  }
}

__device__ __forceinline__ void store(uint16_t* tile, const Stage& st) {
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int c = threadIdx.x + kThreads * j;
    if (c < kT * kChunks)
      *reinterpret_cast<u32x4_t*>(tile + (c / kChunks) * kRS + (c % kChunks) * 8) = st.r[j];
  }
}

}  // namespace

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_mfma_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][kT * kRS];
  __shared__ __attribute__((aligned(16))) float xbuf[8][16][64];

  const DevTask t = a.tasks[blockIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int hg = wave >> 1, dh = wave & 1;
  const int end = min(t.end, a.seq_lens[t.b]);
  const int32_t* ptab = a.page_table + (int64_t)t.b * a.max_pages;
  // head blocks of this wave that exist (H_q may be below 128)
  const bool hb_ok[2] = {32 * hg < a.H_q, 32 * hg + 16 < a.H_q};

  // Q^T operand: lane owns head 32hg + 16hb + n; k-slots of step ks are dims
  // 288 dh + 32 ks + 8 g .. +7.
  u32x4_t qf[2][kKs];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hg + 16 * hb + n;
    const uint16_t* qp = a.q + ((int64_t)t.q_row * a.H_q + min(head, a.H_q - 1)) * kD + 288 * dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      qf[hb][ks] = hb_ok[hb] ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : u32x4_t{0, 0, 0, 0};
  }

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4_t o[kNb][2];
#pragma unroll
  for (int nb = 0; nb < kNb; ++nb) o[nb][0] = o[nb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stage st;
  int t0 = t.lo;
  if (t0 < end) {
    fetch(a, ptab, end, t0, st);
    store(tiles[0], st);
    if (t0 + kT < end) fetch(a, ptab, end, t0 + kT, st);
  }
  int buf = 0;
  for (; t0 < end; t0 += kT, buf ^= 1) {
    __syncthreads();  // tiles[buf] written; everyone is done with tiles[buf ^ 1]
    if (t0 + kT < end) {
      store(tiles[buf ^ 1], st);
      if (t0 + 2 * kT < end) fetch(a, ptab, end, t0 + 2 * kT, st);
    }
    const uint16_t* tile = tiles[buf];

    // ---- partial scores over this wave's 288 qk dims ----
    f32x4_t s[2][2];  // [token block][head block]
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) s[blk][0] = s[blk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // row i of token block blk is token 8(i/4) + 4 blk + i%4, so that a lane's
    // outputs (rows 4g..4g+3 of both blocks) are the 8 consecutive tokens 8g..8g+7
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int tok = 8 * (n >> 2) + 4 * blk + (n & 3);
        const u32x4_t ka =
            *reinterpret_cast<const u32x4_t*>(tile + tok * kRS + 288 * dh + 32 * ks + 8 * g);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          if (hb_ok[hb]) s[blk][hb] = mfma16(ka, qf[hb][ks], s[blk][hb]);
      }
    }
    // ---- add the partner wave's half of the scores ----
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) xbuf[wave][8 * blk + 4 * hb + e][lane] = s[blk][hb][e];
    __syncthreads();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[blk][hb][e] += xbuf[wave ^ 1][8 * blk + 4 * hb + e][lane];

    // ---- online softmax per head (log2 domain) ----
    const bool tail = t0 + kT > end;
    u32x4_t pf[2];
    float alpha[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float sv[8];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = t0 + 8 * g + 4 * blk + e;
          const float x = s[blk][hb][e] * a.scale_log2;
          sv[4 * blk + e] = (!tail || tok < end) ? x : -INFINITY;
        }
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m[hb], mt);
      alpha[hb] = fast_exp2(m[hb] - mn);
      m[hb] = mn;
      float p[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(sv[i] - mn);
        ps += p[i];
      }
      l[hb] = l[hb] * alpha[hb] + ps;
      pf[hb] = u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                       pack_bf16x2(p[6], p[7])};
    }

    // ---- O^T over this wave's 256 value dims ----
    // transposing reads: lane (g, i) addresses token 8g + i/4 (+4), dims d0 + 4(i%4)
    const uint16_t* vrow = tile + (8 * g + (n >> 2)) * kRS + 256 * dh + 4 * (n & 3);
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
      const u32x2_t lo = tr_read(vrow + 16 * nb);
      const u32x2_t hi = tr_read(vrow + 4 * kRS + 16 * nb);
      const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (!hb_ok[hb]) continue;
        o[nb][hb] *= alpha[hb];
        o[nb][hb] = mfma16(va, pf[hb], o[nb][hb]);
      }
    }
  }

  // ---- epilogue: normalise and write this wave's (heads, dims) block ----
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (!hb_ok[hb]) continue;
    float lt = l[hb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int head = 32 * hg + 16 * hb + n;
    if (head >= a.H_q) continue;
    const bool empty = m[hb] == -INFINITY;
    const float inv = empty ? 0.f : 1.f / lt;
    const int64_t row = (int64_t)t.out_row + head;
    float* orow = a.o_part + row * kDv + 256 * dh + 4 * g;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb)
      *reinterpret_cast<f32x4_t*>(orow + 16 * nb) = o[nb][hb] * inv;
    if (dh == 0 && g == 0) a.lse_part[row] = empty ? -INFINITY : (m[hb] + fast_log2(lt)) * kLn2;
  }
}

hipError_t launch_mla_mfma(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  if (d.head_dim_qk != kD || d.head_dim_v != kDv || d.num_kv_heads != 1 || d.dtype != SKV_BF16)
    return hipErrorInvalidValue;
  if (L.num_tasks == 0) return hipSuccess;
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(L.q);
  a.kv = static_cast<const uint8_t*>(L.k_pages);
  a.page_table = L.page_table;
  a.seq_lens = L.seq_lens;
  a.tasks = reinterpret_cast<const DevTask*>(static_cast<const uint8_t*>(L.workspace) + L.tasks_off);
  a.err_flag = reinterpret_cast<int32_t*>(const_cast<void*>(L.workspace));
  a.o_part = L.o_part;
  a.lse_part = L.lse_part;
  a.H_q = d.num_q_heads;
  a.page_shift = __builtin_ctz((unsigned)d.page_size);
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.scale_log2 = d.softmax_scale * kLog2e;
  hipLaunchKernelGGL(mla_mfma_kernel, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
  return hipGetLastError();
}

}  // namespace skv
