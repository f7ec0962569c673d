// Paged split-KV partial attention for absorbed multi-head latent attention
// (bf16, up to 128 query heads sharing one 576-wide latent row per token whose
// first 512 entries are the value), on the matrix cores.
//
// Shapes follow SPLASH sections 2-3: KV bytes per token L(d_c + d_r)b with
// d_c = 512 and d_r = 64; the attention at a request's owner computes rows
// [N_r, H, d_c + d_r] and returns width d_c. One work-group runs one task: all
// heads of one query token over the KV range [lo, end) of one split, so each
// latent row is read from HBM once per task and shared by every head (the
// reason MLA decode is matrix-core work: ~242 flop per KV byte).
//
// Work split: 8 waves (2 per SIMD); wave w owns head group hg = w / 2 (32
// heads) and dimension half dh = w % 2. For a 32-token tile staged in LDS it
// computes with v_mfma_f32_16x16x32_bf16
//   S^T[32 tok x 32 heads] partial over its 288 of the 576 qk dims
//       (two token blocks x two 16-head blocks),
// adds the partner wave's half through LDS (both then hold identical full
// scores and softmax state), and
//   O^T[256 dims x 32 heads] += V^T[256 x 32 tok] * P^T[32 tok x 32 heads]
// over its 256 of the 512 value dims. Every output element has one owner wave.
// Each lane owns one head per head block in both outputs, so the softmax needs
// no data movement beyond two lane shuffles. The V^T operand comes from the
// row-major latent tile through the gfx950 transposing LDS read
// (ds_read_b64_tr_b16: within each 16 lanes, lane i addresses row i/4, columns
// 4(i%4)..+3 of a 4 x 16 block and lane n receives column n of its four rows),
// so the tile is stored in LDS once. Tiles stream HBM -> LDS with the gfx950
// LDS DMA (global_load_lds_dwordx4: lane i's 16 bytes land at the wave's LDS
// base + 16 i) into a ring of three buffers, without staging registers.
// Softmax weights enter P*V as one bf16 term (|error| <= 2^-9 max|V| per
// weight, within the bf16 tolerance for latent values; this kernel is
// matrix-bound, unlike the GQA one). Waves 0-3 and 4-7 (the two waves of each
// SIMD) run the per-tile matrix and vector phases one barrier step apart, so
// that the softmax of one overlaps the matrix work of the other.
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
// LDS tile layout, in 16-byte slots: rows of 74 slots (72 of data, 2 of pad)
// in groups of 8 rows followed by one pad slot. With 32 four-byte banks, the
// row stride of 296 dwords (8 mod 32) makes the transposing V reads (4 rows x 4
// eight-byte column groups per 16 lanes) conflict-free, and the extra slot per
// 8 rows keeps the K reads of rows t and t + 8 (same 8-lane pass) apart.
constexpr int kSlots = 74;                       // slots per LDS row
constexpr int kRS = kSlots * 8;                  // LDS row stride in bf16 (592)
constexpr int kGroupSlots = 8 * kSlots + 1;      // 593 slots per group of 8 rows
constexpr int kGS = kGroupSlots * 8;             // group stride in bf16
constexpr int kTileSlots = (kT / 8) * kGroupSlots;  // 2372
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaPerTile = (kTileSlots + 63) / 64;               // 38 wave-instructions
constexpr int kDmaPerWave = (kDmaPerTile + kWaves - 1) / kWaves;  // 5 for waves 0-5, else 4
constexpr int kKs = kD / 2 / 32;  // 32-wide k-steps per qk dimension half (9)
constexpr int kNb = kDv / 2 / 16; // 16-dim output blocks per value dimension half (16)

typedef short __attribute__((__vector_size__(4 * sizeof(short)))) s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
// Page-table reads go through the constant address space: the table is not
// written while the kernel runs, so they become scalar loads, which are
// counted apart from the LDS DMA and never make the tile loop wait for it.
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2_t tr_read(const uint16_t* lds_ptr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_ptr));
  return __builtin_bit_cast(u32x2_t, v);
}

// One wave-wide LDS DMA: each active lane's 16 bytes at `src` land at
// dst + 16 * lane. Issued as inline assembly so that the compiler does not
// track it: its own wait insertion would otherwise drain every DMA in flight
// before each read of a different ring buffer (it cannot tell the buffers
// apart). The tile loop orders these writes itself with vmcnt waits, which
// stay correct for the compiler's own loads because vector-memory counters
// retire in order. M0 carries the LDS base; one wait state separates its write
// from the DMA.
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint16_t* dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_t*)dst;
  __asm__ __volatile__(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
      : "memory", "m0");
}

// The same with a wave-uniform 64-bit base and a 32-bit per-lane byte offset
// (the instruction's scalar-address form: no 64-bit vector arithmetic).
__device__ __forceinline__ void lds_dma16_sbase(const uint8_t* base, uint32_t off, uint16_t* dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_t*)dst;
  __asm__ __volatile__(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
      : "memory", "m0");
}

// Byte offset, within a run of 32 consecutive latent rows, of the 16 bytes
// that slot 64 inst + lane of a tile holds (pad slots: offset 0, a harmless
// valid read that lands in a slot nothing reads).
__device__ __forceinline__ uint32_t slot_offset(int inst, int lane) {
  const int s = 64 * inst + lane;
  const int grp = s / kGroupSlots, rem = s - grp * kGroupSlots;
  const int rig = rem / kSlots, ch = rem - rig * kSlots;   // rig = 8 for the group pad
  const bool data = rig < 8 && ch < kD / 8;
  return data ? (uint32_t)((8 * grp + rig) * kD * 2 + ch * 16) : 0u;
}

// Issue this wave's share of the DMA of the 32-token tile at t0 into `tile`.
// Every slot of the tile is fetched by exactly one lane, so each wave issues a
// fixed number of DMA instructions per tile (5 for waves 0-5, 4 for 6-7),
// which the vmcnt waits of the main loop rely on. Rows at or past `end`, pad
// slots and rows of an out-of-range page read page 0 instead (always valid);
// their scores are masked and their values zeroed where they are used. Page ids
// are wave-uniform scalars: a tile starts at a multiple of 32 tokens, so it
// spans one page (P >= 32) or two (P = 16). They are read from the page table
// one tile ahead of their use (see TilePages), so that the scalar-load latency
// is not paid at every tile.
struct TilePages {
  int pid0, pid1;
};
__device__ __forceinline__ TilePages load_pages(const MlaArgs& a, const_i32_t* ptab, int end, int t0) {
  // the second index does not depend on the first load, so neither load
  // makes the wave wait before the ids are used
  const int last = (end - 1) >> a.page_shift;   // never index past the request's pages
  const int i0 = min(t0 >> a.page_shift, last);
  const int i1 = (a.page_shift == 4 && t0 + 16 < end) ? min((t0 + 16) >> 4, last) : i0;
  return TilePages{ptab[i0], ptab[i1]};
}
__device__ __forceinline__ void issue_tile(const MlaArgs& a, TilePages pg, int end, int t0,
                                           uint16_t* tile, int wave, int lane, const uint32_t* soff) {
  // Recompute the per-lane slot arithmetic at every call: hoisted out of the
  // tile loop it would occupy registers the kernel does not have, and the
  // reload of a spilled address would wait for the DMAs issued before it.
  __asm__ __volatile__("" : "+v"(lane));
  const int P = 1 << a.page_shift;
  const int pid0 = pg.pid0, pid1 = pg.pid1;
  const bool ok0 = pid0 >= 0 && pid0 < a.num_pages;
  const bool ok1 = pid1 >= 0 && pid1 < a.num_pages;
  if ((!ok0 || !ok1) && lane == 0) raise_error(a.err_flag, 1);
  if (P >= 32) {
    // The tile is 32 consecutive rows of one page: a scalar base plus the
    // lane's fixed offset. Rows past `end` are read from the same (valid)
    // page and masked where they are used.
    const uint8_t* base = a.kv + (ok0 ? ((int64_t)pid0 * P + (t0 & (P - 1))) * (kD * 2) : 0);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int inst = wave + kWaves * j;
      if (inst >= kDmaPerTile) break;   // wave-uniform
      const uint32_t off = soff[64 * j + lane];
      if (inst == kDmaPerTile - 1) {   // the only instruction with lanes past the tile
        if (64 * inst + lane < kTileSlots) lds_dma16_sbase(base, off, tile + 64 * 8 * inst);
      } else {
        lds_dma16_sbase(base, off, tile + 64 * 8 * inst);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int inst = wave + kWaves * j;
    if (inst >= kDmaPerTile) break;   // wave-uniform
    const int s = 64 * inst + lane;
    const int grp = s / kGroupSlots, rem = s - grp * kGroupSlots;
    const int rig = rem / kSlots, ch = rem - rig * kSlots;   // rig = 8 for the group pad
    const int row = 8 * grp + rig;
    const int tok = t0 + row;
    const bool hi = P == 16 && row >= 16;
    const int pid = hi ? pid1 : pid0;
    const bool ok = rig < 8 && ch < kD / 8 && tok < end && (hi ? ok1 : ok0);
    const uint8_t* src = ok ? a.kv + (((int64_t)pid * P + (tok & (P - 1))) * kD + ch * 8) * 2 : a.kv;
    if (s < kTileSlots)   // only the last instruction has lanes past the tile
      lds_dma16(src, tile + 64 * 8 * inst);
  }
}

}  // namespace

// Workgroup barrier without a memory fence: LDS writes are ordered by the
// explicit counter waits before it (a fenced barrier would also drain the LDS
// DMA of the tiles still in flight).
__device__ __forceinline__ void bare_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_mfma_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ring[3][kTileSlots * 8];
  __shared__ __attribute__((aligned(16))) f32x4_t xbuf[kWaves][4][64];
  __shared__ uint32_t soff_lds[kWaves][kDmaPerWave * 64];

  const DevTask t = a.tasks[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int hg = wave >> 1, dh = wave & 1;
  const int end = min(t.end, a.seq_lens[t.b]);
  const_i32_t* ptab = (const_i32_t*)(a.page_table + (int64_t)t.b * a.max_pages);

  // Q^T operand: lane owns head 32 hg + 16 hb + n (heads past H_q compute on a
  // copy of the last head and are not written); k-slots of step ks are dims
  // 288 dh + 32 ks + 8 g .. +7.
  u32x4_t qf[2][kKs];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = min(32 * hg + 16 * hb + n, a.H_q - 1);
    const uint16_t* qp = a.q + ((int64_t)t.q_row * a.H_q + head) * kD + 288 * dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qf[hb][ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
  }

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4_t o[kNb][2];
#pragma unroll
  for (int nb = 0; nb < kNb; ++nb) o[nb][0] = o[nb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Q has landed before the first DMA: otherwise the compiler places its wait
  // at the first use, inside the tile loop, where it would drain the DMA ring
  __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
  const int ntiles = end > t.lo ? (end - t.lo + kT - 1) / kT : 0;
  // the lanes' fixed DMA offsets (used when a page holds 32 or more tokens),
  // kept in LDS: registers are fully used; each wave reads only its own
  uint32_t* soff = soff_lds[wave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) soff[64 * j + lane] = slot_offset(wave + kWaves * j, lane);
  // Schedule. A tile's work is a matrix phase M(k) = [P*V of tile k-1, partial
  // scores of tile k] and a vector phase V(k) = [partner's half of the scores,
  // online softmax of tile k]. Waves 0-3 run M(0) V(0) M(1) V(1) ... M(n), one
  // phase per step; waves 4-7 (the other wave of each SIMD) run the same one
  // step later, so on every SIMD one wave feeds the matrix core while the
  // other works on the vector ALU. Steps are separated by work-group barriers
  // (2n + 2 steps, every wave passes each). Tile k + 1 is fetched during steps
  // 2k and 2k + 1 into the ring buffer that tile k - 2 left (its last reader,
  // the second group's M(k - 1), ran in step 2k - 1); every wave drains its
  // DMAs before the barrier of each even step.
  const int grp = wave >> 2;
  if (ntiles > 0) issue_tile(a, load_pages(a, ptab, end, t.lo), end, t.lo, ring[0], wave, lane, soff);
  TilePages pg_next = load_pages(a, ptab, end, t.lo + kT);   // pages of the next tile to fetch
  f32x4_t s[2][2];   // scores of the current tile: [token block][head block]
  u32x4_t pf[2];     // softmax weights of the last tile, bf16 (P^T operand)

  auto matrix_phase = [&](const int k) {
    if (k >= 1) {
      // ---- O^T over this wave's 256 value dims, tile k - 1 ----
      const int tp = t.lo + (k - 1) * kT;
      const bool ptail = tp + kT > end;
      const int nvalid = ptail ? end - (tp + 8 * g) : 8;   // valid tokens among 8g..8g+7
      // transposing reads: lane (g, i) addresses token 8g + i/4 (+4), dims d0 + 4(i%4)
      const uint16_t* vrow = ring[(k + 2) % 3] + g * kGS + (n >> 2) * kRS + 256 * dh + 4 * (n & 3);
#pragma unroll
      for (int nb = 0; nb < kNb; ++nb) {
        const u32x2_t lo = tr_read(vrow + 16 * nb);
        const u32x2_t hi = tr_read(vrow + 4 * kRS + 16 * nb);
        u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
        if (ptail) {   // values of tokens past `end` (unfetched or stale rows) are zeroed
#pragma unroll
          for (int e = 0; e < 4; ++e)
            va[e] &= (2 * e + 1 < nvalid ? 0xFFFF0000u : 0u) | (2 * e < nvalid ? 0x0000FFFFu : 0u);
        }
        o[nb][0] = mfma16(va, pf[0], o[nb][0]);
        o[nb][1] = mfma16(va, pf[1], o[nb][1]);
        if (nb % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k < ntiles) {
      // ---- partial scores over this wave's 288 qk dims, tile k ----
      const uint16_t* tile = ring[k % 3];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) s[blk][0] = s[blk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // row i of token block blk is token 8(i/4) + 4 blk + i%4, so that a lane's
      // outputs (rows 4g..4g+3 of both blocks) are the 8 consecutive tokens 8g..8g+7
      const uint16_t* krow0 = tile + (n >> 2) * kGS + (n & 3) * kRS + 288 * dh + 8 * g;
      // operand reads one k-step ahead of their MFMAs (two-stage register ring)
      u32x4_t kb[2][2];
      auto kread = [&](int ks, u32x4_t (&dst)[2]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          dst[blk] = *reinterpret_cast<const u32x4_t*>(krow0 + 4 * blk * kRS + 32 * ks);
      };
      kread(0, kb[0]);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        if (ks + 1 < kKs) kread(ks + 1, kb[(ks + 1) % 2]);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          s[blk][0] = mfma16(kb[ks % 2][blk], qf[0][ks], s[blk][0]);
          s[blk][1] = mfma16(kb[ks % 2][blk], qf[1][ks], s[blk][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // publish this half for the partner wave (read after the next barrier)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) xbuf[wave][2 * blk + hb][lane] = s[blk][hb];
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the writes are done
    }
  };

  auto vector_phase = [&](const int k) {
    const int t0 = t.lo + k * kT;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) s[blk][hb] += xbuf[wave ^ 1][2 * blk + hb][lane];
    // ---- online softmax per head (log2 domain) ----
    // The running reference m only moves when a tile's maximum exceeds it by
    // more than 8 (a factor 256): weights exp2(s - m) then stay <= 256, the
    // accumulators are rescaled only on those (rare) tiles, and the common
    // path leaves them to the matrix cores. The result is the same softmax.
    if (t0 + kT > end) {   // tokens at or past `end` take no part: score -inf, weight 0
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t0 + 8 * g + 4 * blk + e >= end) s[blk][hb][e] = -INFINITY;
    }
    float alpha[2] = {1.f, 1.f};
    bool bump = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      // the maximum of the raw scores, scaled (scaling by a positive factor
      // and rounding are monotone, so this is the maximum of the scaled scores)
      float mt = fmaxf(fmaxf(fmaxf(s[0][hb][0], s[0][hb][1]), fmaxf(s[0][hb][2], s[0][hb][3])),
                       fmaxf(fmaxf(s[1][hb][0], s[1][hb][1]), fmaxf(s[1][hb][2], s[1][hb][3])));
      mt = max_xor32(max_xor16(mt)) * a.scale_log2;
      if (mt > m[hb] + 8.f) {   // also true on the first tile (m = -inf)
        alpha[hb] = fast_exp2(m[hb] - mt);
        l[hb] *= alpha[hb];
        m[hb] = mt;
        bump = true;
      }
      float ps = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[blk][hb][e] = fast_exp2(fmaf(s[blk][hb][e], a.scale_log2, -m[hb]));
          ps += s[blk][hb][e];
        }
      l[hb] += ps;
      pf[hb] = u32x4_t{pack_bf16x2(s[0][hb][0], s[0][hb][1]), pack_bf16x2(s[0][hb][2], s[0][hb][3]),
                       pack_bf16x2(s[1][hb][0], s[1][hb][1]), pack_bf16x2(s[1][hb][2], s[1][hb][3])};
    }
    // P*V of tile k runs in the next matrix phase, after the accumulators of
    // tiles up to k - 1 are rescaled to the new reference
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
      for (int nb = 0; nb < kNb; ++nb) {
        o[nb][0] *= alpha[0];
        o[nb][1] *= alpha[1];
      }
    }
  };

  // even steps: drain this wave's DMAs (tile step/2 has then landed for all),
  // synchronise, start the next tile's DMA and read the page ids of the one after
  auto even_barrier = [&](const int step) {
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
    bare_barrier();
    const int k1 = step / 2 + 1;
    if (k1 < ntiles) {
      issue_tile(a, pg_next, end, t.lo + k1 * kT, ring[k1 % 3], wave, lane, soff);
      pg_next = load_pages(a, ptab, end, t.lo + (k1 + 1) * kT);   // clamped: always a valid entry
    }
  };
  // Each group runs its own copy of the loop, so that only its own live state
  // crosses the loop edge (the weights for group 0, the scores for group 1).
  if (ntiles > 0) {
    if (grp == 0) {
      for (int k = 0; k < ntiles; ++k) {
        even_barrier(2 * k);
        matrix_phase(k);
        bare_barrier();
        vector_phase(k);
      }
      even_barrier(2 * ntiles);
      matrix_phase(ntiles);
      bare_barrier();
    } else {
      even_barrier(0);
      for (int k = 0; k < ntiles; ++k) {
        bare_barrier();
        matrix_phase(k);
        even_barrier(2 * k + 2);
        vector_phase(k);
      }
      bare_barrier();
      matrix_phase(ntiles);
    }
  }

  // ---- epilogue: normalise and write this wave's (heads, dims) block ----
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float lt = l[hb];
    lt = sum_xor32(sum_xor16(lt));
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
