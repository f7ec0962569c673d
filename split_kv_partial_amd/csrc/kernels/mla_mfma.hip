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
// Work split: 4 waves, one per SIMD, each with the SIMD's whole register file
// (512 per lane; the output accumulators sit in the accumulation registers).
// Wave w owns heads 32w..32w+31 over all dimensions, so waves share nothing
// but the KV tile. For a 32-token tile staged in LDS it computes with
// v_mfma_f32_16x16x32_bf16
//   S^T[32 tok x 32 heads] = K[32 x 576] Q^T[576 x 32 heads]
//       (two token blocks x two 16-head blocks),
// the online softmax, and
//   O^T[512 dims x 32 heads] += V^T[512 x 32 tok] P^T[32 tok x 32 heads].
// Each lane owns one head per head block and the same eight tokens in both
// products, so the softmax needs no data movement beyond two lane shuffles.
// The V^T operand comes from the row-major latent tile through the gfx950
// transposing LDS read (ds_read_b64_tr_b16: within each 16 lanes, lane i
// addresses row i/4, columns 4(i%4)..+3 of a 4 x 16 block and lane n receives
// column n of its four rows), so the tile is stored in LDS once. Tiles stream
// HBM -> LDS with the gfx950 LDS DMA (global_load_lds_dwordx4: lane i's 16
// bytes land at the wave's LDS base + 16 i) into a ring of four buffers, each
// tile issued three tiles ahead of its use, without staging registers.
// Softmax weights enter P*V as one bf16 term (|error| <= 2^-9 max|V| per
// weight, within the bf16 tolerance for latent values).
#include <type_traits>

#include "device_common.hpp"
#include "fused.hpp"
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
  const float* kv_scale;   // FP8 rows: float32 scale per page (NULL for bf16 rows)
  int32_t H_q, page_shift, max_pages, num_pages;
  float scale_log2;
};

namespace {

constexpr int kD = 576;          // qk width: 512 latent + 64 rope
constexpr int kDv = 512;         // value width (the latent)
constexpr int kT = 32;           // tokens per tile
constexpr int kRowSlots = kD / 8;             // 16-byte slots per latent row (72)
constexpr int kRowBytes = kD * 2;             // 1152
constexpr int kTileSlots = kT * kRowSlots;    // 2304
constexpr int kTileElems = kTileSlots * 8;    // bf16 per LDS tile buffer
constexpr int kTileBytes = kTileSlots * 16;   // 36,864
constexpr int kBuf = 4;                       // LDS ring depth
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaPerTile = kTileSlots / 64;        // 36 wave-instructions
constexpr int kDmaPerWave = kDmaPerTile / kWaves;   // 9
static_assert(kTileSlots % 64 == 0 && kDmaPerTile % kWaves == 0, "whole DMA instructions per wave");
constexpr int kKs = kD / 32;     // 32-wide k-steps of the scores (18)
constexpr int kNb = kDv / 16;    // 16-dim output blocks (32)
constexpr int kKd = 4;           // K operand reads in flight, in k-steps
constexpr int kVd = 12;          // V operand reads in flight, in output blocks

// LDS tile layout: row r (token t0 + r) holds its 72 slots unpadded, chunk c
// of the row at slot 72 r + (c ^ swz(r)). LDS bank structure of gfx950, as
// measured with the bank-conflict counter: 64 four-byte banks (a 256-byte
// line of 16 slots); a 16-byte read serves 16 lanes per cycle, lanes 8h..8h+7
// of a 16-lane group g together with the other half of group g ^ 1 (lanes
// 0-7 with 24-31, 8-15 with 16-23); an 8-byte transposing read serves 32
// lanes per cycle. Row parity separates the two halves of a bank line
// (72 r mod 16 = 8 (r % 2)) and the XOR of bits 1 and 3 of r spreads the rows
// of one parity, so that the K reads (per cycle: 16 rows, chunks 4 ks + g and
// 4 ks + (g ^ 1)) and the V reads (8 rows at two adjacent chunks) touch every
// bank once.
__device__ __forceinline__ int swz(int r) { return (r & 2) | ((r >> 1) & 4); }

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

// The four score MFMAs of one k-step, s[blk][hb] += K[blk] Q[hb], as inline
// assembly: the compiler gives every MFMA result of a kernel the same register
// kind, and the 256 output accumulators need all the accumulation registers,
// so the scores are kept in vector registers this way. The compiler does not
// see these as MFMAs when it inserts wait states: the operands here are only
// written by LDS loads (the K fragments), by the global loads of Q before the
// tile loop and by these MFMAs (chained accumulation needs no wait states),
// the first step starts from zero accumulators instead of registers cleared
// by a vector ALU instruction and begins with three wait states anyway, and
// scores_ready() below covers the MFMA -> vector ALU distance.
template <bool kFirst>
__device__ __forceinline__ void qk_step(f32x4_t (&s)[2][2], const u32x4_t (&kf)[2], u32x4_t q0,
                                        u32x4_t q1) {
  if (kFirst)
    __asm__("s_nop 2\n\t"
            "v_mfma_f32_16x16x32_bf16 %0, %4, %6, 0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %4, %7, 0\n\t"
            "v_mfma_f32_16x16x32_bf16 %2, %5, %6, 0\n\t"
            "v_mfma_f32_16x16x32_bf16 %3, %5, %7, 0"
            : "=&v"(s[0][0]), "=&v"(s[0][1]), "=&v"(s[1][0]), "=&v"(s[1][1])
            : "v"(kf[0]), "v"(kf[1]), "v"(q0), "v"(q1));
  else
    __asm__("v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
            "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
            "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3"
            : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1])
            : "v"(kf[0]), "v"(kf[1]), "v"(q0), "v"(q1));
}
// max(a, b, c) in one instruction. (The compiler's fmaxf would first quiet
// each operand, since it cannot see that the scores are never signalling
// NaNs.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Twenty wait states between the last score MFMA and the first vector ALU
// read of the scores (more than an MFMA of this shape needs).
__device__ __forceinline__ void scores_ready(f32x4_t (&s)[2][2]) {
  __asm__ __volatile__("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                       : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}

__device__ __forceinline__ u32x2_t tr_read(const uint8_t* lds_ptr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_ptr));
  return __builtin_bit_cast(u32x2_t, v);
}

// One of this wave's nine LDS DMAs of a tile: instruction j moves each lane's
// 16 bytes to LDS byte lds + 4096 j + 16 lane (the wave's 1 KB blocks wave,
// wave + 4, ... of the tile). Inline assembly, so that the compiler does not
// track them: its own wait insertion would otherwise drain every DMA in
// flight before each read of a different ring buffer (it cannot tell the
// buffers apart). The tile loop orders these writes itself with vmcnt waits,
// which stay correct for the compiler's own loads because vector-memory
// counters retire in order. M0 carries the LDS address; one wait state
// separates its write from the DMA that reads it.
template <int J>
__device__ __forceinline__ void dma_sbase(const uint8_t* base, uint32_t off, uint32_t lds) {
  __asm__ __volatile__(
      "s_add_u32 m0, %[l], %[o4k]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o], %[b] nt"
      :
      : [l] "s"(lds), [o4k] "i"(J * 4096), [b] "s"(base), [o] "v"(off)
      : "memory", "m0");
}
template <int J>
__device__ __forceinline__ void dma_vaddr(const uint8_t* src, uint32_t lds) {
  __asm__ __volatile__(
      "s_add_u32 m0, %[l], %[o4k]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[p], off nt"
      :
      : [l] "s"(lds), [o4k] "i"(J * 4096), [p] "v"(src)
      : "memory", "m0");
}
static_assert(kDmaPerWave == 9 && kWaves * 1024 == 4096, "the DMA helpers assume 9 per wave, 4 waves");

// Byte offset, within a run of 32 consecutive latent rows, of the 16 bytes
// that LDS slot 64 inst + lane of a tile holds (the inverse of the layout).
__device__ __forceinline__ uint32_t slot_offset(int inst, int lane) {
  const int s = 64 * inst + lane;
  const int r = s / kRowSlots;
  const int c = (s - r * kRowSlots) ^ swz(r);
  return (uint32_t)(r * kRowBytes + c * 16);
}

// Page ids of the tile at t0, wave-uniform scalars: a tile starts at a
// multiple of 32 tokens, so it spans one page (P >= 32) or two (P = 16). Read
// from the page table well ahead of their use, so that the scalar-load latency
// is not paid at every tile. Indices are clamped to the request's last page,
// so every id read is a real entry of the request.
struct TilePages {
  int pid0, pid1;
};
__device__ __forceinline__ TilePages load_pages(const MlaArgs& a, const_i32_t* ptab, int end, int t0) {
  // the second index does not depend on the first load, so neither load
  // makes the wave wait before the ids are used
  const int last = (end - 1) >> a.page_shift;
  const int i0 = min(t0 >> a.page_shift, last);
  const int i1 = a.page_shift == 4 ? min((t0 + 16) >> 4, last) : i0;
  return TilePages{ptab[i0], ptab[i1]};
}

// This wave's share (9 instructions, a fixed count the vmcnt waits of the
// tile loop rely on) of the DMA of the 32-token tile at t0: prepare() takes
// the page bases and reads the lanes' offsets, issue<J>() sends instruction
// J. Every slot of the tile is fetched by exactly one lane. Rows at or past
// `end` are read from the same (valid) page and masked where they are used.
// An id outside the page pool is never dereferenced: it is reported, page 0
// stands in for it, and the task's state is written as NaN.
template <bool kSinglePage>   // P >= 32: the tile is 32 consecutive rows of one page
struct TileDma {
  const uint8_t* base0;   // the tile's first row (P >= 32) or first page (P = 16)
  const uint8_t* base1;   // P = 16: the second page
  uint32_t off[kDmaPerWave];
  uint32_t lds;

  // Returns true if a page id of the tile is outside the pool (the same for
  // every wave: the ids are wave-uniform scalars of the same tile).
  __device__ __forceinline__ bool prepare(const MlaArgs& a, TilePages pg, int t0, uint32_t lds_addr,
                                          int lane, const uint32_t* soff) {
    const int P = 1 << a.page_shift;
    const bool ok0 = pg.pid0 >= 0 && pg.pid0 < a.num_pages;
    const bool ok1 = pg.pid1 >= 0 && pg.pid1 < a.num_pages;
    if ((!ok0 || !ok1) && lane == 0) raise_error(a.err_flag, kErrPageId);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) off[j] = soff[64 * j + lane];
    lds = __builtin_amdgcn_readfirstlane(lds_addr);
    if (kSinglePage) {
      base0 = a.kv + (ok0 ? ((int64_t)pg.pid0 * P + (t0 & (P - 1))) * kRowBytes : 0);
      base1 = base0;
    } else {
      base0 = a.kv + (ok0 ? (int64_t)pg.pid0 * 16 * kRowBytes : 0);
      base1 = a.kv + (ok1 ? (int64_t)pg.pid1 * 16 * kRowBytes : 0);
    }
    return !ok0 || !ok1;
  }
  template <int J>
  __device__ __forceinline__ void issue() const {
    if (kSinglePage) {
      dma_sbase<J>(base0, off[J], lds);
    } else {   // 16-token pages: rows 16..31 come from the second page
      const bool hi = off[J] >= 16u * kRowBytes;
      dma_vaddr<J>(hi ? base1 + (off[J] - 16u * kRowBytes) : base0 + off[J], lds);
    }
  }
  __device__ __forceinline__ void issue_all() const {
    issue<0>(); issue<1>(); issue<2>(); issue<3>(); issue<4>();
    issue<5>(); issue<6>(); issue<7>(); issue<8>();
  }
};

}  // namespace

// Workgroup barrier without a memory fence: LDS writes are ordered by the
// explicit counter waits before it (a fenced barrier would also drain the LDS
// DMA of the tiles still in flight).
__device__ __forceinline__ void bare_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding) that wait for the vector-memory counter
// only: at most 0, 9 or 18 of this wave's DMA instructions still in flight.
constexpr int kWaitVm0 = 0x3f70;
constexpr int kWaitVm9 = 0x3f70 | 9;
constexpr int kWaitVm18 = 0x3f70 | (18 & 15) | ((18 >> 4) << 14);
static_assert(2 * kDmaPerWave == 18 && kBuf == 4, "vmcnt immediates assume 9 DMAs per tile, 4 buffers");

// LDS of one work-group: the tile ring, each wave's DMA offsets, and the
// restart decision of the softmax.
struct MlaShared {
  __attribute__((aligned(16))) uint16_t ring[kBuf][kTileElems];
  uint32_t soff_lds[kWaves][kDmaPerWave * 64];
  int restart_pass;   // the last pass in which some head overflowed
};

// One task: all heads of one query token over the KV range [lo, end) of one
// split, written as the split's partial state. Every wave of the work-group
// runs it; it begins and ends with the ring unused.
template <bool kSinglePage>
__device__ __forceinline__ void mla_task(const MlaArgs& a, const DevTask& task, MlaShared& sh) {
  // the task's fields as wave-uniform values (scalar registers), whatever the
  // caller's code lets the compiler prove: the DMA takes its base address
  // from scalar registers
  DevTask t;
  t.b = __builtin_amdgcn_readfirstlane(task.b);
  t.kvh = 0;
  t.lo = __builtin_amdgcn_readfirstlane(task.lo);
  t.end = __builtin_amdgcn_readfirstlane(task.end);
  t.q_row = __builtin_amdgcn_readfirstlane(task.q_row);
  t.out_row = __builtin_amdgcn_readfirstlane(task.out_row);
  t.seq_len = __builtin_amdgcn_readfirstlane(task.seq_len);
  t.pad = 0;
  auto& ring = sh.ring;
  auto& soff_lds = sh.soff_lds;
  int& restart_pass = sh.restart_pass;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  if (a.seq_lens[t.b] != t.seq_len) {
    // the device lengths are not the ones the plan was built from: no KV is
    // read and the state is NaN (uniform over the work-group: one task)
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrSeqLen);
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.H_q, kDv);
    return;
  }
  const int end = t.end;
  const_i32_t* ptab = (const_i32_t*)(a.page_table + (int64_t)t.b * a.max_pages);

  // Q^T operand: lane owns head 32 wave + 16 hb + n (heads past H_q compute on
  // a copy of the last head and are not written); k-slots of step ks are dims
  // 32 ks + 8 g .. +7.
  u32x4_t qf[2][kKs];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = min(32 * wave + 16 * hb + n, a.H_q - 1);
    const uint16_t* qp = a.q + ((int64_t)t.q_row * a.H_q + head) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qf[hb][ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
  }
  // Q has landed before the first DMA: otherwise the compiler places its wait
  // at the first use, inside the tile loop, where it would drain the DMA ring
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  const int ntiles = end > t.lo ? (end - t.lo + kT - 1) / kT : 0;
  // the lanes' fixed DMA offsets, kept in LDS; each wave reads only its own
  uint32_t* soff = soff_lds[wave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) soff[64 * j + lane] = slot_offset(wave + kWaves * j, lane);
  if (threadIdx.x == 0) restart_pass = 0;
  // LDS byte address of this wave's first DMA block in ring buffer 0
  const uint32_t ring_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&ring[0][0]) + 1024u * wave;

  // Per-lane byte offsets of the operand reads within a tile buffer.
  // K (A operand of the scores): lane (g, n) reads row 8(n/4) + 4 blk + n%4 of
  // token block blk, so that its outputs (rows 4g..4g+3 of both blocks) are
  // the 8 consecutive tokens 8g..8g+7, and chunk 4 ks + g of step ks; with the
  // layout's XOR that is slot base + 4 ks + 4 h2 (even ks) or - 4 h2 (odd ks).
  uint32_t ke[2], ko[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int r = 8 * (n >> 2) + 4 * blk + (n & 3);
    const int h = swz(r);
    const int base = kRowSlots * r + (g ^ (h & 3));
    ke[blk] = 16u * (uint32_t)(base + 4 * (h >> 2));
    ko[blk] = 16u * (uint32_t)(base - 4 * (h >> 2));
  }
  // V (transposing reads): lane (g, n) addresses row 8g + n/4 (and + 4),
  // columns 16 nb + 4(n%4)..+3, i.e. half n%2 of chunk 2 nb + (n%4)/2; with
  // the XOR the slot is 72 r + ((n%4)/2 ^ h0) + 2 ((nb%4) ^ h12) + 8 (nb/4).
  uint32_t va4[4];
  {
    const int r = 8 * g + (n >> 2);
    const int h = swz(r);
    const int vb = kRowSlots * r + (((n & 3) >> 1) ^ (h & 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) va4[j] = 16u * (uint32_t)(vb + 2 * (j ^ (h >> 1))) + 8u * (n & 1);
  }

  // Online softmax without rescaling. The reference m of a head is the
  // maximum of its first tile, and the weights exp2(s - m) of later tokens
  // may exceed 1: up to 2^64 they are exact in range for bf16 and the fp32
  // sums (a split holds at most 2^31 tokens of bounded values), and the
  // normalisation at the end gives the same softmax. After the first tile
  // each lane only compares its own scores with the fixed reference (no
  // cross-lane step per tile) and keeps its running maximum. A score above
  // m + 64 makes the whole work-group run the split again, with references
  // raised to the largest scores of the pass, which no score exceeds: at most
  // one restart (ordinary attention scores never trigger one; the scale is
  // positive, checked on the host). A second pass that still overflows can
  // only come from rounding of absurdly scaled scores: it is reported and the
  // state written as NaN instead of running a third pass. The
  // accumulators are thus never rewritten inside the tile loop, which keeps
  // them in the accumulation registers.
  float m[2] = {0.f, 0.f};             // references (log2 domain, scaled)
  float thr[2] = {INFINITY, INFINITY};  // raw score above which m + 64 is exceeded
  float mr[2] = {-INFINITY, -INFINITY}; // the lane's running raw maximum
  // a head's reference: the maximum of its raw scores so far over the lanes
  // holding it, scaled (a positive scale and rounding are monotone)
  auto set_reference = [&](int hb) {
    m[hb] = max_xor32(max_xor16(mr[hb])) * a.scale_log2;
    thr[hb] = (m[hb] + 64.f) / a.scale_log2;
  };
  float l[2];
  f32x4_t o[kNb][2];
  bool bad_page = false;    // some page id of the split is outside the pool
  bool range_err = false;   // scores beyond what one restart can represent
  for (int pass = 1;; ++pass) {
    bool over = false;   // some head of this wave overflowed in this pass
    l[0] = l[1] = 0.f;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) o[nb][0] = o[nb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Ring: tile k sits in buffer k % 4. Tiles 0-2 are issued up front; tile
    // k + 3 at the top of iteration k, into the buffer tile k - 1 left (every
    // wave has passed that iteration's barrier, so its reads are done).
    TilePages pg{0, 0};
    if (ntiles > 0) pg = load_pages(a, ptab, end, t.lo);
#pragma unroll
    for (int j = 0; j < kBuf - 1; ++j) {
      if (j < ntiles) {
        TileDma<kSinglePage> d;
        bad_page |= d.prepare(a, pg, t.lo + j * kT, ring_lds + j * kTileBytes, lane, soff);
        d.issue_all();
        pg = load_pages(a, ptab, end, t.lo + (j + 1) * kT);   // clamped: always a valid entry
      }
    }

    for (int k = 0; k < ntiles; ++k) {
      // tile k has landed for this wave (its DMAs retire in order), then for all
      const int ahead = ntiles - 1 - k;   // tiles after k already issued: min(2, ahead)
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(kWaitVm18);
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(kWaitVm9);
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      bare_barrier();
      // the DMA of tile k + 3, spread over the score MFMAs below (issued back
      // to back, the nine instructions stall the wave)
      const bool fetch = k + kBuf - 1 < ntiles;
      TileDma<kSinglePage> d;   // prepared always (the page ids are clamped), issued if fetch
      bad_page |= d.prepare(a, pg, t.lo + (k + kBuf - 1) * kT,
                            ring_lds + ((k + kBuf - 1) % kBuf) * kTileBytes, lane, soff);
      if (fetch) pg = load_pages(a, ptab, end, t.lo + (k + kBuf) * kT);
      uint16_t* tile = ring[k % kBuf];
      const uint8_t* lb = reinterpret_cast<const uint8_t*>(tile);
      const int t0 = t.lo + k * kT;
      const bool tail = t0 + kT > end;
      if (tail) {
        // rows past `end` hold stale data of the page (possibly not finite):
        // zero them, so that their (zero) weights meet zero values
        const int r0 = end - t0;
        for (int sl = kRowSlots * r0 + threadIdx.x; sl < kTileSlots; sl += kThreads)
          reinterpret_cast<u32x4_t*>(tile)[sl] = u32x4_t{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        bare_barrier();
      }

      // ---- scores S^T of tile k over all 576 dims ----
      f32x4_t s[2][2];
      auto qk = [&](auto fetch_tag) {
        constexpr bool kFetch = decltype(fetch_tag)::value;
        u32x4_t kb[kKd][2];
        auto kread = [&](int ks, u32x4_t (&dst)[2]) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            dst[blk] = *reinterpret_cast<const u32x4_t*>(lb + ((ks & 1) ? ko[blk] : ke[blk]) + 64 * ks);
        };
#pragma unroll
        for (int i = 0; i < kKd - 1; ++i) {
          kread(i, kb[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          if (ks + kKd - 1 < kKs) kread(ks + kKd - 1, kb[(ks + kKd - 1) % kKd]);
          if (ks == 0) qk_step<true>(s, kb[0], qf[0][0], qf[1][0]);
          else qk_step<false>(s, kb[ks % kKd], qf[0][ks], qf[1][ks]);
          if (kFetch && ks % 2 == 1) {
            switch (ks / 2) {
              case 0: d.template issue<0>(); break;
              case 1: d.template issue<1>(); break;
              case 2: d.template issue<2>(); break;
              case 3: d.template issue<3>(); break;
              case 4: d.template issue<4>(); break;
              case 5: d.template issue<5>(); break;
              case 6: d.template issue<6>(); break;
              case 7: d.template issue<7>(); break;
              default: d.template issue<8>(); break;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (fetch) qk(std::true_type{});
      else qk(std::false_type{});
      scores_ready(s);

      // ---- softmax weights (log2 domain) ----
      if (tail) {   // tokens at or past `end` take no part: score -inf, weight 0
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (t0 + 8 * g + 4 * blk + e >= end) s[blk][hb][e] = -INFINITY;
      }
      u32x4_t pf[2];   // weights of tile k, bf16 (P^T operand)
      const bool first = k == 0 && pass == 1;   // the tile that fixes the references
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        // the lane's running maximum of its raw scores in this pass
        mr[hb] = max3f(max3f(s[0][hb][0], s[0][hb][1], s[0][hb][2]),
                       max3f(s[0][hb][3], s[1][hb][0], s[1][hb][1]),
                       max3f(s[1][hb][2], s[1][hb][3], mr[hb]));
        if (first) set_reference(hb);
        over = over || mr[hb] > thr[hb];
        // the row sums add the fp32 weights (their bf16 roundings would cost
        // the exported log-sum-exp up to 2^-9)
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

      // ---- O^T += V^T P^T over all 512 value dims, tile k ----
      {
        u32x4_t vb[kVd];
        auto vread = [&](int nb, u32x4_t& dst) {
          const uint8_t* p = lb + va4[nb & 3] + 128 * (nb >> 2);
          const u32x2_t lo = tr_read(p);
          const u32x2_t hi = tr_read(p + 4 * kRowSlots * 16);   // rows + 4
          dst = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        };
#pragma unroll
        for (int i = 0; i < kVd - 1; ++i) {
          vread(i, vb[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb) {
          if (nb + kVd - 1 < kNb) vread(nb + kVd - 1, vb[(nb + kVd - 1) % kVd]);
          o[nb][0] = mfma16(vb[nb % kVd], pf[0], o[nb][0]);
          o[nb][1] = mfma16(vb[nb % kVd], pf[1], o[nb][1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every wave has finished the pass (and its DMAs) before the decision;
    // the flag is only written by this pass, so it needs no reset
    if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) restart_pass = pass;
    __builtin_amdgcn_s_waitcnt(kWaitVm0 & 0xc07f);   // vmcnt(0) lgkmcnt(0)
    bare_barrier();
    if (restart_pass != pass) break;
    if (pass == 2) {
      // the second pass starts from the first pass's maxima, which no score
      // of the split exceeds: an overflow here means scores whose scaled
      // values fp32 cannot separate (an absurd scale); report, do not loop
      range_err = true;
      if (threadIdx.x == 0) raise_error(a.err_flag, kErrRange);
      break;
    }
    // the next pass starts from the largest scores this one saw
    set_reference(0);
    set_reference(1);
  }
  if (bad_page || range_err) {   // uniform: every wave saw the same ids and flag
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.H_q, kDv);
    return;
  }

  // ---- epilogue: normalise and write this wave's 32 heads ----
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float lt = l[hb];
    lt = sum_xor32(sum_xor16(lt));
    const int head = 32 * wave + 16 * hb + n;
    if (head >= a.H_q) continue;
    const bool empty = ntiles == 0;
    const float inv = empty ? 0.f : 1.f / lt;
    const int64_t row = (int64_t)t.out_row + head;
    float* orow = a.o_part + row * kDv + 4 * g;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb)
      *reinterpret_cast<f32x4_t*>(orow + 16 * nb) = o[nb][hb] * inv;
    if (g == 0) a.lse_part[row] = empty ? -INFINITY : (m[hb] + fast_log2(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) latent rows: [num_pages][P][576] one-byte codes with one
// float32 scale per page (SPLASH appendix C.1 serves its MLA backend from an
// FP8 E4M3 KV cache). A stored entry is its code's E4M3 value times the page's
// scale; the value of a token is the first 512 entries of its row, under the
// same scale. The tile loop is the bf16 one: each 32-token tile is read by the
// products from a bf16 tile in the same swizzled LDS layout. The codes stream
// HBM -> LDS in 64-token tiles (36 KB: the same nine 1 KB DMAs per wave as a
// bf16 tile, so two compute tiles per DMA tile) into a ring of two, and the
// work-group converts each 32-token half once into one of two bf16 tiles
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value is a bf16
// value, so the codes are decoded exactly) one tile ahead of its products.
// The page scale multiplies the tile's scores (folded into the exponent's
// multiplier, and into the running maximum) and the softmax weights before
// they are packed for P*V, while the normaliser sums the unscaled weights:
// o = sum_j p_j (s_j c_j) / sum_j p_j with c_j the decoded codes.
// Schedule: FP8 tile F (F >= 2) is sent at iteration 2F - 3 into the ring slot
// that FP8 tile F - 2 left (both its halves converted by then), and is
// converted from iteration 2F - 1 on; iteration k converts tile k + 1 and
// computes tile k.
// ---------------------------------------------------------------------------
constexpr int kF8Tokens = 64;                      // tokens per FP8 DMA tile
constexpr int kF8TileBytes = kF8Tokens * kD;       // 36,864: 36 DMA blocks of 1 KB
constexpr int kF8HalfBytes = kT * kD;              // 18,432: the codes of one 32-token tile
constexpr int kCvt = kT * kRowSlots / kThreads;    // 8-code chunks per lane per tile (9)
static_assert(kF8TileBytes == kDmaPerTile * 1024 && kCvt == kDmaPerWave, "FP8 tiles reuse the DMA shape");

typedef const __attribute__((address_space(4))) float const_f32_t;

struct MlaShared8 {
  __attribute__((aligned(16))) uint8_t f8[2][kF8TileBytes];
  __attribute__((aligned(16))) uint16_t bf[2][kTileElems];
  // per lane, its nine chunks of a tile: byte offset of the codes within the
  // 32-token half (low 16 bits) and of the bf16 slot within the tile (high)
  uint32_t cvt_lds[kWaves][kCvt * 64];
  int restart_pass;
};

// Chunk i of lane `lane` of wave `wave`: wave w converts rows 8w..8w+7 of a
// tile, its lanes taking the 576 chunks of 8 codes in order.
__device__ __forceinline__ uint32_t cvt_entry(int wave, int i, int lane) {
  const int idx = 64 * i + lane;
  const int r = 8 * wave + idx / kRowSlots, c = idx % kRowSlots;
  const uint32_t src = (uint32_t)(r * kD + 8 * c);
  const uint32_t dst = (uint32_t)(16 * (kRowSlots * r + (c ^ swz(r))));
  return src | (dst << 16);
}

// Two E4M3 codes (byte pair kHi of w) as two bf16 in one word, exactly.
template <bool kHi>
__device__ __forceinline__ uint32_t f8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// Decode this lane's nine chunks of one 32-token half of an FP8 tile (codes
// at `half`) into a bf16 tile (`tile`), both in LDS.
__device__ __forceinline__ void convert_tile(const uint8_t* half, uint8_t* tile, const uint32_t* tab, int lane) {
  uint32_t e[kCvt];
#pragma unroll
  for (int i = 0; i < kCvt; ++i) e[i] = tab[64 * i + lane];
  u32x2_t c[kCvt];
#pragma unroll
  for (int i = 0; i < kCvt; ++i) c[i] = *reinterpret_cast<const u32x2_t*>(half + (e[i] & 0xFFFFu));
#pragma unroll
  for (int i = 0; i < kCvt; ++i) {
    const u32x4_t v = {f8x2_to_bf16x2<false>(c[i][0]), f8x2_to_bf16x2<true>(c[i][0]),
                       f8x2_to_bf16x2<false>(c[i][1]), f8x2_to_bf16x2<true>(c[i][1])};
    *reinterpret_cast<u32x4_t*>(tile + (e[i] >> 16)) = v;
  }
}

// This wave's nine DMAs of the 64-token FP8 tile at t0 (a multiple of 64, so
// the tile covers 64 / P whole pages): block b = 4j + wave lies in page
// b / (9P / 16) of the tile at byte (b mod 9P / 16) * 1 KB. Page indices past
// the request's last page are clamped to it (rows past `end` are masked where
// they are used). Returns true if a page id is outside the pool: it is not
// dereferenced (page 0 stands in) and the state is written as NaN.
template <int kP>
__device__ __forceinline__ bool f8_dma(const MlaArgs& a, const_i32_t* ptab, int end, int t0, uint32_t lds,
                                       int wave, uint32_t voff) {
  constexpr int kPages = kF8Tokens / kP;
  constexpr int kBpp = 9 * kP / 16;   // 1 KB blocks per page
  const int last = (end - 1) / kP;
  const uint8_t* base[kPages];
  bool bad = false;
#pragma unroll
  for (int pg = 0; pg < kPages; ++pg) {
    const int pid = ptab[min(t0 / kP + pg, last)];
    const bool ok = pid >= 0 && pid < a.num_pages;
    bad |= !ok;
    base[pg] = a.kv + (ok ? (int64_t)pid * (kP * kD) : 0);
  }
  if (bad && (threadIdx.x & 63) == 0) raise_error(a.err_flag, kErrPageId);
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int b = 4 * j + wave;
    const int pg = kPages == 1 ? 0 : b / kBpp;
    const uint8_t* src = base[0];
#pragma unroll
    for (int q = 1; q < kPages; ++q)
      if (pg == q) src = base[q];
    src += (b - pg * kBpp) * 1024;
    switch (j) {
      case 0: dma_sbase<0>(src, voff, lds); break;
      case 1: dma_sbase<1>(src, voff, lds); break;
      case 2: dma_sbase<2>(src, voff, lds); break;
      case 3: dma_sbase<3>(src, voff, lds); break;
      case 4: dma_sbase<4>(src, voff, lds); break;
      case 5: dma_sbase<5>(src, voff, lds); break;
      case 6: dma_sbase<6>(src, voff, lds); break;
      case 7: dma_sbase<7>(src, voff, lds); break;
      default: dma_sbase<8>(src, voff, lds); break;
    }
  }
  return bad;
}

template <int kP>
__device__ __forceinline__ void mla_task_f8(const MlaArgs& a, const DevTask& task, MlaShared8& sh) {
  DevTask t;
  t.b = __builtin_amdgcn_readfirstlane(task.b);
  t.kvh = 0;
  t.lo = __builtin_amdgcn_readfirstlane(task.lo);
  t.end = __builtin_amdgcn_readfirstlane(task.end);
  t.q_row = __builtin_amdgcn_readfirstlane(task.q_row);
  t.out_row = __builtin_amdgcn_readfirstlane(task.out_row);
  t.seq_len = __builtin_amdgcn_readfirstlane(task.seq_len);
  t.pad = 0;
  int& restart_pass = sh.restart_pass;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  if (a.seq_lens[t.b] != t.seq_len) {
    if (threadIdx.x == 0) raise_error(a.err_flag, kErrSeqLen);
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.H_q, kDv);
    return;
  }
  const int end = t.end;
  const_i32_t* ptab = (const_i32_t*)(a.page_table + (int64_t)t.b * a.max_pages);
  const_f32_t* pscale = (const_f32_t*)a.kv_scale;

  u32x4_t qf[2][kKs];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = min(32 * wave + 16 * hb + n, a.H_q - 1);
    const uint16_t* qp = a.q + ((int64_t)t.q_row * a.H_q + head) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qf[hb][ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  const int ntiles = end > t.lo ? (end - t.lo + kT - 1) / kT : 0;
  const int nf = (ntiles + 1) / 2;   // FP8 DMA tiles
  uint32_t* tab = sh.cvt_lds[wave];
#pragma unroll
  for (int i = 0; i < kCvt; ++i) tab[64 * i + lane] = cvt_entry(wave, i, lane);
  if (threadIdx.x == 0) restart_pass = 0;
  const uint32_t f8_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sh.f8[0][0]);
  const uint32_t dma_lds = f8_lds + 1024u * wave;   // this wave's first DMA block in slot 0
  const uint32_t voff = 16u * lane;

  // operand read offsets: those of the bf16 kernel
  uint32_t ke[2], ko[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int r = 8 * (n >> 2) + 4 * blk + (n & 3);
    const int h = swz(r);
    const int base = kRowSlots * r + (g ^ (h & 3));
    ke[blk] = 16u * (uint32_t)(base + 4 * (h >> 2));
    ko[blk] = 16u * (uint32_t)(base - 4 * (h >> 2));
  }
  uint32_t va4[4];
  {
    const int r = 8 * g + (n >> 2);
    const int h = swz(r);
    const int vb = kRowSlots * r + (((n & 3) >> 1) ^ (h & 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) va4[j] = 16u * (uint32_t)(vb + 2 * (j ^ (h >> 1))) + 8u * (n & 1);
  }

  float m[2] = {0.f, 0.f};
  float thr[2] = {INFINITY, INFINITY};
  float mr[2] = {-INFINITY, -INFINITY};   // the lane's running maximum of scaled raw scores
  auto set_reference = [&](int hb) {
    m[hb] = max_xor32(max_xor16(mr[hb])) * a.scale_log2;
    thr[hb] = (m[hb] + 64.f) / a.scale_log2;
  };
  float l[2];
  f32x4_t o[kNb][2];
  bool bad_page = false;
  bool range_err = false;
  for (int pass = 1;; ++pass) {
    bool over = false;
    l[0] = l[1] = 0.f;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) o[nb][0] = o[nb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // FP8 tiles 0 and 1, then tile 0's first half converted
#pragma unroll
    for (int f = 0; f < 2; ++f)
      if (f < nf) bad_page |= f8_dma<kP>(a, ptab, end, t.lo + f * kF8Tokens, dma_lds + f * kF8TileBytes, wave, voff);
    if (ntiles > 0) {
      if (nf > 1) __builtin_amdgcn_s_waitcnt(kWaitVm9);
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      bare_barrier();
      convert_tile(&sh.f8[0][0], reinterpret_cast<uint8_t*>(&sh.bf[0][0]), tab, lane);
    }

    for (int k = 0; k < ntiles; ++k) {
      // odd k: FP8 tile (k + 1) / 2, which tile k + 1 is converted from, has
      // landed for this wave (no later DMA is in flight); every k: tile k's
      // conversion is written (LDS counter) before the barrier
      if (k & 1) __builtin_amdgcn_s_waitcnt(kWaitVm0 & 0xc07f);
      else __builtin_amdgcn_s_waitcnt(0xc07f);
      bare_barrier();
      const int F = (k + 3) / 2;   // the FP8 tile sent at this (odd) iteration
      if ((k & 1) && F < nf)
        bad_page |= f8_dma<kP>(a, ptab, end, t.lo + F * kF8Tokens, dma_lds + (F & 1) * kF8TileBytes, wave, voff);
      // page scale(s) of tile k: one page (P >= 32) or two (P = 16; a lane's
      // eight tokens lie in one 16-token half); ids outside the pool read page
      // 0's scale (the state is NaN anyway)
      const int t0 = t.lo + k * kT;
      float sc;
      {
        const int last = (end - 1) / kP;
        const int p0 = ptab[min(t0 / kP, last)];
        const float s0 = pscale[(p0 >= 0 && p0 < a.num_pages) ? p0 : 0];
        if (kP == 16) {
          const int p1 = ptab[min(t0 / kP + 1, last)];
          const float s1 = pscale[(p1 >= 0 && p1 < a.num_pages) ? p1 : 0];
          sc = g < 2 ? s0 : s1;
        } else {
          sc = s0;
        }
      }
      uint16_t* tile = sh.bf[k & 1];
      const uint8_t* lb = reinterpret_cast<const uint8_t*>(tile);
      const bool tail = t0 + kT > end;
      if (tail) {
        const int r0 = end - t0;
        for (int sl = kRowSlots * r0 + threadIdx.x; sl < kTileSlots; sl += kThreads)
          reinterpret_cast<u32x4_t*>(tile)[sl] = u32x4_t{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(0xc07f);
        bare_barrier();
      }
      // tile k + 1's codes into the other bf16 tile (its last reader, tile
      // k - 1, finished before this iteration's barrier)
      if (k + 1 < ntiles)
        convert_tile(&sh.f8[(k + 1) / 2 & 1][((k + 1) & 1) * kF8HalfBytes],
                     reinterpret_cast<uint8_t*>(&sh.bf[(k + 1) & 1][0]), tab, lane);

      // ---- scores S^T of tile k over all 576 dims ----
      f32x4_t s[2][2];
      {
        u32x4_t kb[kKd][2];
        auto kread = [&](int ks, u32x4_t (&dst)[2]) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            dst[blk] = *reinterpret_cast<const u32x4_t*>(lb + ((ks & 1) ? ko[blk] : ke[blk]) + 64 * ks);
        };
#pragma unroll
        for (int i = 0; i < kKd - 1; ++i) {
          kread(i, kb[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          if (ks + kKd - 1 < kKs) kread(ks + kKd - 1, kb[(ks + kKd - 1) % kKd]);
          if (ks == 0) qk_step<true>(s, kb[0], qf[0][0], qf[1][0]);
          else qk_step<false>(s, kb[ks % kKd], qf[0][ks], qf[1][ks]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      scores_ready(s);

      if (tail) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (t0 + 8 * g + 4 * blk + e >= end) s[blk][hb][e] = -INFINITY;
      }
      u32x4_t pf[2];
      const bool first = k == 0 && pass == 1;
      const float mul = a.scale_log2 * sc;   // raw score -> log2 domain, page scale included
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float tmax = max3f(max3f(s[0][hb][0], s[0][hb][1], s[0][hb][2]),
                                 max3f(s[0][hb][3], s[1][hb][0], s[1][hb][1]),
                                 max3f(s[1][hb][2], s[1][hb][3], s[1][hb][3]));
        mr[hb] = max3f(tmax * sc, mr[hb], mr[hb]);   // scaled raw scores (sc > 0 keeps the order)
        if (first) set_reference(hb);
        over = over || mr[hb] > thr[hb];
        float ps = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[blk][hb][e] = fast_exp2(fmaf(s[blk][hb][e], mul, -m[hb]));
            ps += s[blk][hb][e];
          }
        l[hb] += ps;
        // the weights times the page scale meet the decoded codes in P*V
        pf[hb] = u32x4_t{pack_bf16x2(s[0][hb][0] * sc, s[0][hb][1] * sc), pack_bf16x2(s[0][hb][2] * sc, s[0][hb][3] * sc),
                         pack_bf16x2(s[1][hb][0] * sc, s[1][hb][1] * sc), pack_bf16x2(s[1][hb][2] * sc, s[1][hb][3] * sc)};
      }

      // ---- O^T += V^T P^T over all 512 value dims, tile k ----
      {
        u32x4_t vb[kVd];
        auto vread = [&](int nb, u32x4_t& dst) {
          const uint8_t* p = lb + va4[nb & 3] + 128 * (nb >> 2);
          const u32x2_t lo = tr_read(p);
          const u32x2_t hi = tr_read(p + 4 * kRowSlots * 16);
          dst = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        };
#pragma unroll
        for (int i = 0; i < kVd - 1; ++i) {
          vread(i, vb[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb) {
          if (nb + kVd - 1 < kNb) vread(nb + kVd - 1, vb[(nb + kVd - 1) % kVd]);
          o[nb][0] = mfma16(vb[nb % kVd], pf[0], o[nb][0]);
          o[nb][1] = mfma16(vb[nb % kVd], pf[1], o[nb][1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) restart_pass = pass;
    __builtin_amdgcn_s_waitcnt(kWaitVm0 & 0xc07f);
    bare_barrier();
    if (restart_pass != pass) break;
    if (pass == 2) {
      range_err = true;
      if (threadIdx.x == 0) raise_error(a.err_flag, kErrRange);
      break;
    }
    set_reference(0);
    set_reference(1);
  }
  if (bad_page || range_err) {
    write_nan_state(a.o_part, a.lse_part, t.out_row, a.H_q, kDv);
    return;
  }
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float lt = l[hb];
    lt = sum_xor32(sum_xor16(lt));
    const int head = 32 * wave + 16 * hb + n;
    if (head >= a.H_q) continue;
    const bool empty = ntiles == 0;
    const float inv = empty ? 0.f : 1.f / lt;
    const int64_t row = (int64_t)t.out_row + head;
    float* orow = a.o_part + row * kDv + 4 * g;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb)
      *reinterpret_cast<f32x4_t*>(orow + 16 * nb) = o[nb][hb] * inv;
    if (g == 0) a.lse_part[row] = empty ? -INFINITY : (m[hb] + fast_log2(lt)) * kLn2;
  }
}

template <int kP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_mfma_f8_kernel(MlaArgs a) {
  __shared__ MlaShared8 sh;
  mla_task_f8<kP>(a, a.tasks[blockIdx.x], sh);
}

// One work-group per task, in the plan's queue order.
template <bool kSinglePage>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_mfma_kernel(MlaArgs a) {
  __shared__ MlaShared sh;
  mla_task<kSinglePage>(a, a.tasks[blockIdx.x], sh);
}

// Attention and merge in one launch (fused.hpp): the task, then the
// reduction role when every task has started.
template <bool kSinglePage>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_mfma_fused(MlaArgs a, FusedArgs f) {
  __shared__ MlaShared sh;
  __shared__ int slot;
  count_started(f);
  const DevTask t = a.tasks[blockIdx.x];
  mla_task<kSinglePage>(a, t, sh);
  publish_task(f, t.b);
  if (all_started(f, &slot)) reduce_phase<kDv>(f, a.err_flag);
}

static MlaArgs mla_args(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(L.q);
  a.kv = static_cast<const uint8_t*>(L.k_pages);
  a.page_table = L.page_table;
  a.seq_lens = L.seq_lens;
  a.kv_scale = L.k_scales;
  a.tasks = reinterpret_cast<const DevTask*>(static_cast<const uint8_t*>(L.workspace) + L.tasks_off);
  a.err_flag = reinterpret_cast<int32_t*>(const_cast<void*>(L.workspace));
  a.o_part = L.o_part;
  a.lse_part = L.lse_part;
  a.H_q = d.num_q_heads;
  a.page_shift = __builtin_ctz((unsigned)d.page_size);
  a.max_pages = d.max_pages_per_seq;
  a.num_pages = d.num_pages;
  a.scale_log2 = d.softmax_scale * kLog2e;
  return a;
}

hipError_t launch_mla_mfma_fused(const AttnLaunch& L, const FusedLaunch& F) {
  const skv_attn_desc& d = *L.desc;
  if (d.head_dim_qk != kD || d.head_dim_v != kDv || d.num_kv_heads != 1 || d.dtype != SKV_BF16)
    return hipErrorInvalidValue;
  const MlaArgs a = mla_args(L);
  const FusedArgs f = fused_args(F);
  if (d.page_size >= 32)
    hipLaunchKernelGGL(mla_mfma_fused<true>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a, f);
  else
    hipLaunchKernelGGL(mla_mfma_fused<false>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a, f);
  return hipGetLastError();
}

hipError_t launch_mla_mfma(const AttnLaunch& L) {
  const skv_attn_desc& d = *L.desc;
  if (d.head_dim_qk != kD || d.head_dim_v != kDv || d.num_kv_heads != 1) return hipErrorInvalidValue;
  if (d.dtype == SKV_FP8_E4M3) {
    if (!L.k_scales || L.v_scales != L.k_scales) return hipErrorInvalidValue;
    if (L.num_tasks == 0) return hipSuccess;
    const MlaArgs a = mla_args(L);
    if (d.page_size == 64)
      hipLaunchKernelGGL(mla_mfma_f8_kernel<64>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
    else if (d.page_size == 32)
      hipLaunchKernelGGL(mla_mfma_f8_kernel<32>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
    else
      hipLaunchKernelGGL(mla_mfma_f8_kernel<16>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
    return hipGetLastError();
  }
  if (d.dtype != SKV_BF16) return hipErrorInvalidValue;
  if (L.num_tasks == 0) return hipSuccess;
  const MlaArgs a = mla_args(L);
  if (d.page_size >= 32)
    hipLaunchKernelGGL(mla_mfma_kernel<true>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
  else
    hipLaunchKernelGGL(mla_mfma_kernel<false>, dim3(L.num_tasks), dim3(kThreads), 0, L.stream, a);
  return hipGetLastError();
}

}  // namespace skv
