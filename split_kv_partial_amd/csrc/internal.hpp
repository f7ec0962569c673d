// Internal definitions shared by the host library and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "splitkv.h"

namespace skv {

constexpr int kTileTokens = 64;

// One attention work-group's job: request b, KV head g, query tile qi (tokens
// qi * query_tile .. of the request), split r, KV token range [lo, hi) of the
// split. q_row = global index of the tile's first query token; out_row = state
// row of query head g*G of that token in split r.
struct TaskDesc {
  int32_t b, g, qi, r;
  int32_t lo, hi, q_row, out_row;
};
static_assert(sizeof(TaskDesc) == 32, "task descriptor is 32 bytes");

// Device-side descriptor of one attention work-group (built by the host,
// uploaded in launch order).
struct DevTask {
  int32_t b;        // request
  int32_t kvh;      // KV head
  int32_t lo;       // first KV token of the split (multiple of 64)
  int32_t end;      // one past the last KV token this task may read:
                    // min(split end, visible end of its last query token)
  int32_t q_row;    // global index of the task's first query token
  int32_t out_row;  // state row of the first token's first query head
  int32_t seq_len;  // L_b the plan was built with (checked against seq_lens)
  int32_t ntok;     // query tokens of the task (consecutive)
  int32_t hi;       // end of the split's KV range
  int32_t vis_last; // visible end of the last query token (L_b when not causal);
                    // token j of ntok sees min(hi, vis_last - (ntok - 1 - j) * step)
  int32_t step;     // 1 for causal rows, 0 otherwise
  int32_t pad;
};
static_assert(sizeof(DevTask) == 48, "device task descriptor is 48 bytes");

// Per-request data the merge needs.
struct DevReq {
  int32_t state_row;   // first state row of the request
  int32_t splits;      // s_b
  int32_t rows;        // rows_b = q_lens[b] * H_q
  int32_t out_row;     // first merged-output row of the request
  int32_t tasks;       // attention tasks of the request (the fused launch waits for them)
  int32_t pad[3];
};
static_assert(sizeof(DevReq) == 32, "device request descriptor is 32 bytes");

// One merge unit: `count` consecutive rows of request b starting at row `row`.
struct DevUnit {
  int32_t b, row, count, pad;
};

// Device workspace image: [header 256 B][tasks][reqs][units], each 256-aligned.
struct WsHeader {
  int32_t error_flag;
  int32_t num_tasks, batch, num_units;
  int64_t tasks_off, reqs_off, units_off;
  int32_t pad[54];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// Model parameters as used by the planner (mirrors skv_plan_params).
struct ModelParams {
  int tile_tokens = kTileTokens;
  int slots = 256;
  int warps_per_slot = 4;
  int max_splits = 64;
  int overlap_reduction = 0;
  int balanced_candidates = 1;
  double rho = 0.43, delta_attn = 32.0, delta_red = 2.5, gamma = 0.47;
  double min_gain = 0.10, tile_time_us = 1.08;
};

struct Problem {
  std::vector<int64_t> seq_lens, q_lens;
  int num_kv_heads = 1;
  int rows_per_token = 1;
  int n_ext = 0;
  bool causal = true;
  int query_tile = 1;   // query tokens per attention task
};

struct Evaluation {
  std::vector<int> splits;
  double score = 0, t_attn = 0;
  int64_t n_tasks = 0, total_splits = 0;
  std::vector<int> tail;
};

// Planner entry points (planner.cpp).
int64_t n_tiles(int64_t L, int T);
std::vector<std::pair<int64_t, int64_t>> split_ranges(int64_t L, int s, int T);
void build_tasks(const Problem& pb, const ModelParams& prm,
                 const std::vector<std::vector<std::pair<int64_t, int64_t>>>& ranges,
                 std::vector<TaskDesc>& out, std::vector<double>* costs);
int reduction_run(const Problem& pb, const ModelParams& prm);
Evaluation simulate(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits);
std::vector<int> balanced_plan(const Problem& pb, const ModelParams& prm, int64_t wave_tasks);
// ev_out (optional) receives the evaluation of the returned plan.
std::vector<int> reference_plan(const Problem& pb, const ModelParams& prm, Evaluation* ev_out = nullptr);
std::vector<int> split_limits(const Problem& pb, const ModelParams& prm,
                              const std::vector<int>& ref);
// ref_ev (optional): the evaluation of ref, when the caller has it.
Evaluation plan_search(const Problem& pb, const ModelParams& prm, const std::vector<int>& ref,
                       Evaluation* nosplit_out, const Evaluation* ref_ev = nullptr);

// Kernel launchers (one per kernel file). Return hipSuccess or the launch error.
struct AttnLaunch {
  const skv_attn_desc* desc;
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* workspace;
  float* o_part;
  float* lse_part;
  int num_tasks;
  int64_t tasks_off;   // byte offset of the task descriptors in the workspace
  hipStream_t stream;
  int max_ntok;        // most query tokens of any task (1: one token per task)
  const float* k_scales = nullptr;   // FP8 KV: [num_pages][H_kv] key scales
  const float* v_scales = nullptr;   // FP8 KV: [num_pages][H_kv] value scales
};
hipError_t launch_gqa_valu(const AttnLaunch& a);
hipError_t launch_gqa_mfma(const AttnLaunch& a);
hipError_t launch_mla_mfma(const AttnLaunch& a);

struct MergeLaunch {
  const void* workspace;
  const float* o_part;
  const float* lse_part;
  int n_ext;
  const float* o_ext;
  const float* lse_ext;
  void* o_out;
  int out_bf16;
  float* lse_out;
  int head_dim_v;
  int64_t total_rows;
  int num_units;
  int64_t reqs_off, units_off;   // byte offsets in the workspace
  hipStream_t stream;
  int max_states;                // largest states per row (splits + n_ext)
  int run;                       // rows per merge unit (the planner's run)
};
hipError_t launch_merge(const MergeLaunch& m);

// Attention and merge in one launch. block: the scratch's counters block: the
// merge's kernel arguments (kFusedArgsBytes), then kFusedCounterHead + batch
// counters of kFusedCounterLine int32 each (one 256-byte line per counter),
// all written by launch_fused_setup on the same stream before the launch.
constexpr size_t kFusedArgsBytes = 128;
constexpr int kFusedCounterHead = 3;
constexpr int kFusedCounterLine = 64;
struct FusedLaunch {
  uint8_t* block;
};
hipError_t launch_fused_setup(uint8_t* block, const MergeLaunch& m, int batch, int num_tasks,
                              hipStream_t stream);
hipError_t launch_gqa_valu_fused(const AttnLaunch& a, const FusedLaunch& f);
hipError_t launch_gqa_mfma_fused(const AttnLaunch& a, const FusedLaunch& f);
hipError_t launch_mla_mfma_fused(const AttnLaunch& a, const FusedLaunch& f);
hipError_t launch_hbm_probe(const void* buf, int64_t bytes, uint32_t* out, int blocks, hipStream_t stream);
hipError_t launch_mfma_probe(const void* buf, int64_t bytes, int passes, int blocks, int waves, int mfma_waves,
                             int iters, uint32_t* out, hipStream_t stream);

// Error reporting shared by the entry points: sets the thread-local message
// that skv_last_error returns and gives back st.
skv_status fail(skv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Scratch of the whole-path entry points (byte offsets, 256-aligned): counters
// (4 + batch int32), then the partial states o_part [state_rows][D_v] and
// lse_part [state_rows], float32.
struct ScratchLayout {
  size_t counters_off, o_off, lse_off, total;
};
ScratchLayout scratch_layout(const skv_plan* plan);

// The whole path (partial attention of every split, then the merge) with the
// partial states in `scratch`; validates every argument before any launch.
skv_status decode_attn_impl(const skv_attn_desc* desc, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                            const skv_plan* plan, const void* workspace, void* scratch,
                            size_t scratch_bytes, int32_t n_ext, const float* o_ext, const float* lse_ext,
                            void* o_out, int32_t out_dtype, float* lse_out, void* stream,
                            const float* k_scales = nullptr, const float* v_scales = nullptr);

// Default executor shape of each attention kernel (used by the planner).
// GqaMfmaG8: the matrix-core GQA kernel on groups of 8 (the same kernel, with
// its own planner calibration)
enum class Variant { GqaValu, GqaMfma, GqaMfmaG8, MlaMfma };
struct VariantShape {
  int slots_per_cu;    // concurrent attention work-groups per CU
  int merge_waves_per_cu;
};
VariantShape variant_shape(Variant v);
struct Calibration {
  double rho, delta_attn, delta_red, gamma, tile_time_us;
  int balanced;   // whether proportional plans join the final choice by default
};
Calibration calibration(Variant v);

}  // namespace skv
