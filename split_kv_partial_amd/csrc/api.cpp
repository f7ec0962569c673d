// C ABI of the split-KV partial attention library: argument validation, plan
// construction (critical-wave planner, explicit and fixed-chunk plans),
// workspace images, kernel dispatch and error reporting.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "internal.hpp"

using namespace skv;

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace skv {
skv_status fail(skv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
}  // namespace skv

namespace {

bool is_pow2_page(int p) { return p == 16 || p == 32 || p == 64; }

Variant pick_variant(const skv_attn_desc& d);

// Query tokens per attention task for the kernel the problem selects: the
// bf16 matrix-core GQA kernel takes tiles of consecutive tokens whose rows of
// (token, head) fill its four waves' column blocks (128 rows); the others take
// one token (the MLA kernel's 128 heads already fill a tile).
int query_tile_of(const skv_attn_desc& d) {
  const Variant v = pick_variant(d);
  const int rows = 128;
  if (d.dtype == SKV_FP8_E4M3) return 1;   // FP8 KV runs on the one-token kernel
  if (v == Variant::GqaMfma || v == Variant::GqaMfmaG8)
    return std::max(1, rows / (d.num_q_heads / d.num_kv_heads));
  return 1;
}

// Whether the kernel the problem selects runs tasks of qt query tokens.
bool query_tile_runs(const skv_attn_desc& d, int qt) {
  return qt == 1 || qt <= query_tile_of(d);
}

Variant pick_variant(const skv_attn_desc& d) {
  if (d.mla) return Variant::MlaMfma;
  const int G = d.num_q_heads / d.num_kv_heads;
  const bool bf16_q = d.dtype == SKV_BF16 || d.dtype == SKV_FP8_E4M3;
  if (bf16_q && G >= 16) return Variant::GqaMfma;
  if (bf16_q && G == 8) return Variant::GqaMfmaG8;
  return Variant::GqaValu;
}

// Shape checks shared by planning and compute entry points.
skv_status check_desc(const skv_attn_desc* d) {
  if (!d) return fail(SKV_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1) return fail(SKV_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads)
    return fail(SKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (!is_pow2_page(d->page_size))
    return fail(SKV_ERR_UNSUPPORTED, "page_size must be 16, 32 or 64 (got %d)", d->page_size);
  if (d->max_pages_per_seq < 1) return fail(SKV_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
  if (d->num_pages < 1) return fail(SKV_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (d->dtype != SKV_F32 && d->dtype != SKV_BF16 && d->dtype != SKV_FP8_E4M3)
    return fail(SKV_ERR_INVALID_ARG, "dtype must be SKV_F32, SKV_BF16 or SKV_FP8_E4M3 (got %d)", d->dtype);
  // a positive finite scale (the MLA kernel's overflow threshold divides by it)
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f))
    return fail(SKV_ERR_INVALID_ARG, "softmax_scale must be positive and finite (got %g)",
                (double)d->softmax_scale);
  if (d->causal != 0 && d->causal != 1) return fail(SKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->mla) {
    if (d->mla != 1) return fail(SKV_ERR_INVALID_ARG, "mla must be 0 or 1");
    if (d->num_kv_heads != 1 || d->head_dim_qk != 576 || d->head_dim_v != 512 ||
        (d->dtype != SKV_BF16 && d->dtype != SKV_FP8_E4M3))
      return fail(SKV_ERR_UNSUPPORTED,
                  "MLA needs bf16 or FP8 E4M3 rows, num_kv_heads 1, head_dim_qk 576, head_dim_v 512");
    if (d->num_q_heads % 16 || d->num_q_heads > 128)
      return fail(SKV_ERR_UNSUPPORTED, "MLA needs num_q_heads a multiple of 16, at most 128 (got %d)",
                  d->num_q_heads);
    return SKV_OK;
  }
  if ((d->head_dim_qk != 64 && d->head_dim_qk != 128) || d->head_dim_v != d->head_dim_qk)
    return fail(SKV_ERR_UNSUPPORTED, "GQA needs head_dim_qk = head_dim_v in {64, 128} (got %d, %d)",
                d->head_dim_qk, d->head_dim_v);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->dtype == SKV_FP8_E4M3 && G != 8 && G != 16)
    return fail(SKV_ERR_UNSUPPORTED, "FP8 KV needs GQA groups of 8 or 16 query heads (got %d)", G);
  if (pick_variant(*d) == Variant::GqaMfma) {
    if (G != 16)
      return fail(SKV_ERR_UNSUPPORTED, "bf16 GQA groups of 16 or more query heads must be exactly 16 (got %d)", G);
  } else if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) {
    return fail(SKV_ERR_UNSUPPORTED, "GQA group size must be 1, 2, 4, 8 or 16 (got %d)", G);
  }
  return SKV_OK;
}

skv_status check_lengths(const skv_attn_desc& d, const int32_t* seq_lens, const int32_t* q_lens) {
  if (!seq_lens) return fail(SKV_ERR_INVALID_ARG, "seq_lens is NULL");
  for (int b = 0; b < d.batch; ++b) {
    const int64_t L = seq_lens[b], n = q_lens ? q_lens[b] : 1;
    if (n < 1) return fail(SKV_ERR_INVALID_ARG, "q_lens[%d] = %lld must be >= 1", b, (long long)n);
    if (L < n)
      return fail(SKV_ERR_INVALID_ARG, "seq_lens[%d] = %lld is smaller than q_lens[%d] = %lld", b,
                  (long long)L, b, (long long)n);
    if ((L + d.page_size - 1) / d.page_size > d.max_pages_per_seq)
      return fail(SKV_ERR_INVALID_ARG, "seq_lens[%d] = %lld needs more than max_pages_per_seq = %d pages",
                  b, (long long)L, d.max_pages_per_seq);
  }
  return SKV_OK;
}

ModelParams model_params(const skv_attn_desc& d, int num_cu, const skv_plan_params* p) {
  skv_plan_params def;
  skv_plan_params_default(&def);
  if (!p) p = &def;
  const VariantShape vs = variant_shape(pick_variant(d));
  ModelParams m;
  m.tile_tokens = p->tile_tokens;
  const int spc = p->slots_per_cu > 0 ? p->slots_per_cu : vs.slots_per_cu;
  m.slots = num_cu * spc;
  m.warps_per_slot = p->warps_per_slot > 0 ? p->warps_per_slot
                                           : std::max(1, vs.merge_waves_per_cu / spc);
  m.max_splits = p->max_splits;
  m.overlap_reduction = p->overlap_reduction;
  m.balanced_candidates = p->balanced_candidates >= 0 ? p->balanced_candidates
                                                      : calibration(pick_variant(d)).balanced;
  m.min_gain = p->min_gain;
  if (p->use_calibration) {
    const Calibration c = calibration(pick_variant(d));
    m.rho = c.rho;
    m.delta_attn = c.delta_attn;
    m.delta_red = c.delta_red;
    m.gamma = c.gamma;
    m.tile_time_us = c.tile_time_us;
  } else {
    m.rho = p->rho;
    m.delta_attn = p->delta_attn;
    m.delta_red = p->delta_red;
    m.gamma = p->gamma;
    m.tile_time_us = p->tile_time_us;
  }
  return m;
}

skv_status check_params(const skv_plan_params* p) {
  if (!p) return SKV_OK;
  if (p->tile_tokens != kTileTokens) return fail(SKV_ERR_UNSUPPORTED, "tile_tokens must be 64");
  if (p->max_splits < 1 || p->max_splits > 64) return fail(SKV_ERR_INVALID_ARG, "max_splits must be in [1, 64]");
  if (p->slots_per_cu < 0 || p->warps_per_slot < 0) return fail(SKV_ERR_INVALID_ARG, "negative slot counts");
  if (p->use_calibration != 0 && p->use_calibration != 1)
    return fail(SKV_ERR_INVALID_ARG, "use_calibration must be 0 or 1");
  if (p->balanced_candidates < -1 || p->balanced_candidates > 1)
    return fail(SKV_ERR_INVALID_ARG, "balanced_candidates must be -1, 0 or 1");
  if (p->overlap_reduction != 0 && p->overlap_reduction != 1)
    return fail(SKV_ERR_INVALID_ARG, "overlap_reduction must be 0 or 1");
  if (p->query_tile < 0 || p->query_tile > 128)
    return fail(SKV_ERR_INVALID_ARG, "query_tile must be in [0, 128] (got %d)", p->query_tile);
  if (!(p->rho > 0) || !(p->delta_attn >= 0) || !(p->delta_red >= 0) || !(p->gamma >= 0) ||
      !(p->min_gain >= 0 && p->min_gain < 1))
    return fail(SKV_ERR_INVALID_ARG, "model parameters out of range");
  return SKV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct skv_plan {
  skv_attn_desc desc;
  Problem pb;
  ModelParams prm;
  std::vector<std::vector<std::pair<int64_t, int64_t>>> ranges;
  std::vector<int64_t> state_row_offset;  // [B + 1]
  std::vector<TaskDesc> tasks;            // launch order
  std::vector<DevReq> reqs;
  std::vector<DevUnit> units;
  int run = 1;
  int max_ntok = 1;                       // most query tokens of any task
  double score = NAN, t_attn = NAN, nosplit_score = NAN, reference_score = NAN;
  int split_adopted = 0;
  std::vector<uint8_t> image;
  int64_t tasks_off = 0, reqs_off = 0, units_off = 0;
};

namespace {

// Fill tasks, request table, merge units and the workspace image of a plan
// whose ranges are set.
void finish_plan(skv_plan* pl) {
  const skv_attn_desc& d = pl->desc;
  const int B = d.batch;
  const int H = d.num_q_heads, G = d.num_q_heads / d.num_kv_heads;
  pl->state_row_offset.assign(B + 1, 0);
  for (int b = 0; b < B; ++b)
    pl->state_row_offset[b + 1] =
        pl->state_row_offset[b] + (int64_t)pl->ranges[b].size() * pl->pb.q_lens[b] * H;
  build_tasks(pl->pb, pl->prm, pl->ranges, pl->tasks, nullptr);
  std::vector<int64_t> qoff(B + 1, 0);
  for (int b = 0; b < B; ++b) qoff[b + 1] = qoff[b] + pl->pb.q_lens[b];
  std::vector<DevTask> dev(pl->tasks.size());
  const int qt = pl->pb.query_tile;
  for (size_t i = 0; i < pl->tasks.size(); ++i) {
    TaskDesc& t = pl->tasks[i];
    const int64_t L = pl->pb.seq_lens[t.b], n = pl->pb.q_lens[t.b];
    const int64_t rows = n * H;
    const int64_t first = (int64_t)t.qi * qt, last = std::min<int64_t>(n, first + qt) - 1;
    t.out_row = (int32_t)(pl->state_row_offset[t.b] + (int64_t)t.r * rows + first * H + (int64_t)t.g * G);
    const int64_t vis = pl->pb.causal ? L - n + last + 1 : L;
    DevTask& dt = dev[i];
    std::memset(&dt, 0, sizeof dt);
    dt.b = t.b;
    dt.kvh = t.g;
    dt.lo = t.lo;
    dt.end = (int32_t)std::min<int64_t>(t.hi, vis);
    dt.q_row = t.q_row;
    dt.out_row = t.out_row;
    dt.seq_len = (int32_t)L;
    dt.ntok = (int32_t)(last - first + 1);
    pl->max_ntok = std::max(pl->max_ntok, dt.ntok);
    dt.hi = t.hi;
    dt.vis_last = (int32_t)vis;
    dt.step = pl->pb.causal ? 1 : 0;
  }
  pl->reqs.resize(B);
  for (int b = 0; b < B; ++b) {
    pl->reqs[b].state_row = (int32_t)pl->state_row_offset[b];
    pl->reqs[b].splits = (int32_t)pl->ranges[b].size();
    pl->reqs[b].rows = (int32_t)(pl->pb.q_lens[b] * H);
    pl->reqs[b].out_row = (int32_t)(qoff[b] * H);
    pl->reqs[b].tasks = 0;
    pl->reqs[b].pad[0] = pl->reqs[b].pad[1] = pl->reqs[b].pad[2] = 0;
  }
  for (const TaskDesc& t : pl->tasks) ++pl->reqs[t.b].tasks;
  pl->run = reduction_run(pl->pb, pl->prm);
  pl->units.clear();
  for (int b = 0; b < B; ++b) {
    const int rows = pl->reqs[b].rows;
    for (int r = 0; r < rows; r += pl->run) pl->units.push_back({b, r, std::min(pl->run, rows - r), 0});
  }
  pl->tasks_off = sizeof(WsHeader);
  pl->reqs_off = align256(pl->tasks_off + dev.size() * sizeof(DevTask));
  pl->units_off = align256(pl->reqs_off + pl->reqs.size() * sizeof(DevReq));
  const size_t total = align256(pl->units_off + pl->units.size() * sizeof(DevUnit));
  pl->image.assign(total, 0);
  WsHeader hdr;
  std::memset(&hdr, 0, sizeof hdr);
  hdr.num_tasks = (int32_t)dev.size();
  hdr.batch = B;
  hdr.num_units = (int32_t)pl->units.size();
  hdr.tasks_off = pl->tasks_off;
  hdr.reqs_off = pl->reqs_off;
  hdr.units_off = pl->units_off;
  std::memcpy(pl->image.data(), &hdr, sizeof hdr);
  if (!dev.empty()) std::memcpy(pl->image.data() + pl->tasks_off, dev.data(), dev.size() * sizeof(DevTask));
  std::memcpy(pl->image.data() + pl->reqs_off, pl->reqs.data(), pl->reqs.size() * sizeof(DevReq));
  if (!pl->units.empty())
    std::memcpy(pl->image.data() + pl->units_off, pl->units.data(), pl->units.size() * sizeof(DevUnit));
}

skv_status new_plan(const skv_attn_desc* desc, const int32_t* seq_lens, const int32_t* q_lens,
                    int32_t num_cu, int32_t n_ext, const skv_plan_params* params, skv_plan** out,
                    skv_plan** pl_out) {
  if (!out) return fail(SKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  skv_status st = check_desc(desc);
  if (st) return st;
  if ((st = check_lengths(*desc, seq_lens, q_lens))) return st;
  if ((st = check_params(params))) return st;
  if (num_cu < 1) return fail(SKV_ERR_INVALID_ARG, "num_cu must be >= 1");
  if (n_ext < 0 || n_ext > 64) return fail(SKV_ERR_INVALID_ARG, "n_ext must be in [0, 64]");
  skv_plan* pl = new (std::nothrow) skv_plan();
  if (!pl) return fail(SKV_ERR_NO_MEMORY, "plan allocation failed");
  pl->desc = *desc;
  pl->pb.seq_lens.resize(desc->batch);
  pl->pb.q_lens.resize(desc->batch);
  int64_t total_q = 0;
  for (int b = 0; b < desc->batch; ++b) {
    pl->pb.seq_lens[b] = seq_lens[b];
    pl->pb.q_lens[b] = q_lens ? q_lens[b] : 1;
    total_q += pl->pb.q_lens[b];
  }
  if (total_q * desc->num_q_heads * 64 >= ((int64_t)1 << 31)) {
    delete pl;
    return fail(SKV_ERR_UNSUPPORTED, "too many output rows for 32-bit row indices");
  }
  pl->pb.num_kv_heads = desc->num_kv_heads;
  pl->pb.rows_per_token = desc->num_q_heads;
  pl->pb.n_ext = n_ext;
  pl->pb.causal = desc->causal != 0;
  pl->pb.query_tile = params && params->query_tile > 0 ? params->query_tile : query_tile_of(*desc);
  if (!query_tile_runs(*desc, pl->pb.query_tile)) {
    const int qt = pl->pb.query_tile;
    delete pl;
    return fail(SKV_ERR_UNSUPPORTED, "query_tile %d exceeds the %d tokens the selected kernel runs per task",
                qt, query_tile_of(*desc));
  }
  pl->prm = model_params(*desc, num_cu, params);
  *pl_out = pl;
  return SKV_OK;
}

}  // namespace

extern "C" {

void skv_plan_params_default(skv_plan_params* p) {
  if (!p) return;
  std::memset(p, 0, sizeof *p);
  p->tile_tokens = kTileTokens;
  p->slots_per_cu = 0;
  p->warps_per_slot = 0;
  p->max_splits = 64;
  p->overlap_reduction = 0;
  p->use_calibration = 1;
  p->balanced_candidates = -1;
  p->rho = 0.43;
  p->delta_attn = 32.0;
  p->delta_red = 2.5;
  p->gamma = 0.47;
  p->min_gain = 0.10;
  p->tile_time_us = 1.08;
}

skv_status skv_plan_splits(const skv_attn_desc* desc, const int32_t* seq_lens, const int32_t* q_lens,
                           int32_t num_cu, int32_t n_ext, const skv_plan_params* params,
                           const int32_t* ref_splits, skv_plan** out) {
  skv_plan* pl = nullptr;
  skv_status st = new_plan(desc, seq_lens, q_lens, num_cu, n_ext, params, out, &pl);
  if (st) return st;
  try {
    const int B = desc->batch;
    std::vector<int> ref;
    Evaluation ref_ev;
    if (ref_splits) {
      ref.assign(ref_splits, ref_splits + B);
      for (int b = 0; b < B; ++b) {
        const int64_t nt = n_tiles(pl->pb.seq_lens[b], pl->prm.tile_tokens);
        if (ref[b] < 1 || ref[b] > nt || ref[b] > pl->prm.max_splits) {
          delete pl;
          return fail(SKV_ERR_INVALID_ARG, "ref_splits[%d] = %d outside [1, min(tiles, max_splits)]", b, ref[b]);
        }
      }
    } else {
      ref = reference_plan(pl->pb, pl->prm, &ref_ev);
    }
    pl->reference_score = ref_splits ? simulate(pl->pb, pl->prm, ref).score : ref_ev.score;
    Evaluation ns;
    Evaluation ev = plan_search(pl->pb, pl->prm, ref, &ns, ref_splits ? nullptr : &ref_ev);
    pl->score = ev.score;
    pl->t_attn = ev.t_attn;
    pl->nosplit_score = ns.score;
    pl->split_adopted = 0;
    for (int s : ev.splits) pl->split_adopted |= s > 1;
    pl->ranges.resize(B);
    for (int b = 0; b < B; ++b)
      pl->ranges[b] = split_ranges(pl->pb.seq_lens[b], ev.splits[b], pl->prm.tile_tokens);
    finish_plan(pl);
  } catch (const std::bad_alloc&) {
    delete pl;
    return fail(SKV_ERR_NO_MEMORY, "host allocation failed while planning");
  }
  *out = pl;
  return SKV_OK;
}

skv_status skv_plan_from_counts(const skv_attn_desc* desc, const int32_t* seq_lens, const int32_t* q_lens,
                                const int32_t* split_counts, int32_t num_cu, int32_t n_ext,
                                const skv_plan_params* params, skv_plan** out) {
  if (!split_counts) return fail(SKV_ERR_INVALID_ARG, "split_counts is NULL");
  skv_plan* pl = nullptr;
  skv_status st = new_plan(desc, seq_lens, q_lens, num_cu, n_ext, params, out, &pl);
  if (st) return st;
  try {
    const int B = desc->batch;
    std::vector<int> s(split_counts, split_counts + B);
    for (int b = 0; b < B; ++b) {
      const int64_t nt = n_tiles(pl->pb.seq_lens[b], pl->prm.tile_tokens);
      if (s[b] < 1 || s[b] > nt || s[b] > 64) {
        delete pl;
        return fail(SKV_ERR_INVALID_ARG, "split_counts[%d] = %d outside [1, min(tiles, 64)]", b, s[b]);
      }
    }
    Evaluation ev = simulate(pl->pb, pl->prm, s);
    pl->score = ev.score;
    pl->t_attn = ev.t_attn;
    pl->nosplit_score = simulate(pl->pb, pl->prm, std::vector<int>(B, 1)).score;
    pl->ranges.resize(B);
    for (int b = 0; b < B; ++b) {
      pl->ranges[b] = split_ranges(pl->pb.seq_lens[b], s[b], pl->prm.tile_tokens);
      pl->split_adopted |= s[b] > 1;
    }
    finish_plan(pl);
  } catch (const std::bad_alloc&) {
    delete pl;
    return fail(SKV_ERR_NO_MEMORY, "host allocation failed while planning");
  }
  *out = pl;
  return SKV_OK;
}

skv_status skv_plan_fixed_chunks(const skv_attn_desc* desc, const int32_t* seq_lens, const int32_t* q_lens,
                                 int32_t chunk_tokens, int32_t num_cu, skv_plan** out) {
  if (chunk_tokens < kTileTokens || chunk_tokens % kTileTokens)
    return fail(SKV_ERR_INVALID_ARG, "chunk_tokens must be a positive multiple of 64 (got %d)", chunk_tokens);
  skv_plan* pl = nullptr;
  skv_status st = new_plan(desc, seq_lens, q_lens, num_cu, 0, nullptr, out, &pl);
  if (st) return st;
  try {
    const int B = desc->batch;
    pl->ranges.resize(B);
    for (int b = 0; b < B; ++b) {
      const int64_t L = pl->pb.seq_lens[b];
      for (int64_t a = 0; a < L; a += chunk_tokens) pl->ranges[b].emplace_back(a, std::min<int64_t>(L, a + chunk_tokens));
      if (pl->ranges[b].size() > 64) {
        delete pl;
        return fail(SKV_ERR_UNSUPPORTED, "request %d would have %zu chunks (at most 64)", b, pl->ranges[b].size());
      }
      pl->split_adopted |= pl->ranges[b].size() > 1;
    }
    finish_plan(pl);
  } catch (const std::bad_alloc&) {
    delete pl;
    return fail(SKV_ERR_NO_MEMORY, "host allocation failed while planning");
  }
  *out = pl;
  return SKV_OK;
}

skv_status skv_plan_get_info(const skv_plan* pl, skv_plan_info* info) {
  if (!pl || !info) return fail(SKV_ERR_INVALID_ARG, "plan or info is NULL");
  info->batch = pl->desc.batch;
  info->num_tasks = (int32_t)pl->tasks.size();
  int64_t ts = 0;
  for (auto& r : pl->ranges) ts += (int64_t)r.size();
  info->total_splits = (int32_t)ts;
  info->slots = pl->prm.slots;
  info->warps_per_slot = pl->prm.warps_per_slot;
  info->reduction_run = pl->run;
  info->num_units = (int32_t)pl->units.size();
  info->split_adopted = pl->split_adopted;
  info->state_rows = pl->state_row_offset.back();
  int64_t tq = 0;
  for (int64_t n : pl->pb.q_lens) tq += n;
  info->total_rows = tq * pl->desc.num_q_heads;
  info->score = pl->score;
  info->t_attn = pl->t_attn;
  info->nosplit_score = pl->nosplit_score;
  info->rho = pl->prm.rho;
  info->delta_attn = pl->prm.delta_attn;
  info->delta_red = pl->prm.delta_red;
  info->gamma = pl->prm.gamma;
  info->tile_time_us = pl->prm.tile_time_us;
  info->balanced_candidates = pl->prm.balanced_candidates;
  info->query_tile = pl->pb.query_tile;
  info->reference_score = pl->reference_score;
  return SKV_OK;
}

skv_status skv_plan_export(const skv_plan* pl, int32_t* split_counts, int32_t* split_start,
                           int32_t* split_end, int64_t* state_row_offset, int32_t* task_order) {
  if (!pl) return fail(SKV_ERR_INVALID_ARG, "plan is NULL");
  const int B = pl->desc.batch;
  int64_t k = 0;
  for (int b = 0; b < B; ++b) {
    if (split_counts) split_counts[b] = (int32_t)pl->ranges[b].size();
    for (auto& r : pl->ranges[b]) {
      if (split_start) split_start[k] = (int32_t)r.first;
      if (split_end) split_end[k] = (int32_t)r.second;
      ++k;
    }
  }
  if (state_row_offset)
    for (int b = 0; b <= B; ++b) state_row_offset[b] = pl->state_row_offset[b];
  if (task_order)
    for (size_t i = 0; i < pl->tasks.size(); ++i) {
      task_order[4 * i + 0] = pl->tasks[i].b;
      task_order[4 * i + 1] = pl->tasks[i].g;
      task_order[4 * i + 2] = pl->tasks[i].qi;
      task_order[4 * i + 3] = pl->tasks[i].r;
    }
  return SKV_OK;
}

size_t skv_plan_workspace_bytes(const skv_plan* pl) { return pl ? pl->image.size() : 0; }

skv_status skv_plan_upload(const skv_plan* pl, void* ws, size_t bytes, void* stream) {
  if (!pl || !ws) return fail(SKV_ERR_INVALID_ARG, "plan or workspace is NULL");
  if (bytes < pl->image.size())
    return fail(SKV_ERR_NO_MEMORY, "workspace has %zu bytes, the plan needs %zu", bytes, pl->image.size());
  hipError_t e = hipMemcpyAsync(ws, pl->image.data(), pl->image.size(), hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  return SKV_OK;
}

void skv_plan_destroy(skv_plan* pl) { delete pl; }

static skv_status check_plan_matches(const skv_attn_desc* d, const skv_plan* pl) {
  if (!pl) return fail(SKV_ERR_INVALID_ARG, "plan is NULL");
  const skv_attn_desc& p = pl->desc;
  if (d->batch != p.batch || d->num_q_heads != p.num_q_heads || d->num_kv_heads != p.num_kv_heads ||
      d->head_dim_qk != p.head_dim_qk || d->head_dim_v != p.head_dim_v || d->mla != p.mla ||
      d->causal != p.causal || d->page_size != p.page_size || d->dtype != p.dtype)
    return fail(SKV_ERR_PLAN_MISMATCH, "plan was built for a different problem description");
  for (int b = 0; b < d->batch; ++b)
    if ((pl->pb.seq_lens[b] + d->page_size - 1) / d->page_size > d->max_pages_per_seq)
      return fail(SKV_ERR_PLAN_MISMATCH, "plan's seq_lens[%d] exceeds max_pages_per_seq", b);
  if (!query_tile_runs(*d, pl->pb.query_tile))
    return fail(SKV_ERR_UNSUPPORTED, "the kernel for this problem does not run tasks of %d query tokens",
                pl->pb.query_tile);
  return SKV_OK;
}

}  // extern "C"

namespace {

// Argument checks of the attention launch (no launch). FP8 KV takes its
// scales; other storage takes none.
skv_status check_attention(const skv_attn_desc* desc, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                           const skv_plan* plan, const void* workspace, const float* k_scales = nullptr,
                           const float* v_scales = nullptr) {
  skv_status st = check_desc(desc);
  if (st) return st;
  if ((st = check_plan_matches(desc, plan))) return st;
  if (!q || !k_pages || !v_pages || !page_table || !seq_lens || !workspace)
    return fail(SKV_ERR_INVALID_ARG, "a device pointer is NULL");
  if (desc->dtype == SKV_FP8_E4M3 && (!k_scales || !v_scales))
    return fail(SKV_ERR_INVALID_ARG, "FP8 KV needs its key and value scales (skv_decode_attn_partial_fp8)");
  if (desc->dtype != SKV_FP8_E4M3 && (k_scales || v_scales))
    return fail(SKV_ERR_INVALID_ARG, "scales go with FP8 KV only");
  if (desc->mla && v_pages != k_pages)
    return fail(SKV_ERR_INVALID_ARG, "MLA reads values from the key rows: v_pages must equal k_pages");
  if (desc->mla && desc->dtype == SKV_FP8_E4M3 && v_scales != k_scales)
    return fail(SKV_ERR_INVALID_ARG, "FP8 MLA rows have one scale per page: v_scales must equal k_scales");
  return SKV_OK;
}

// Argument checks of the merge launch (no launch).
skv_status check_merge(const skv_attn_desc* desc, const skv_plan* plan, const void* workspace,
                       int32_t n_ext, const float* o_ext, const float* lse_ext, const void* o_out,
                       int32_t out_dtype) {
  skv_status st = check_desc(desc);
  if (st) return st;
  if ((st = check_plan_matches(desc, plan))) return st;
  if (!workspace || !o_out) return fail(SKV_ERR_INVALID_ARG, "a device pointer is NULL");
  if (n_ext < 0 || n_ext > 64) return fail(SKV_ERR_INVALID_ARG, "n_ext must be in [0, 64]");
  if (n_ext > 0 && (!o_ext || !lse_ext)) return fail(SKV_ERR_INVALID_ARG, "external states are NULL");
  if (out_dtype != SKV_F32 && out_dtype != SKV_BF16) return fail(SKV_ERR_INVALID_ARG, "bad out_dtype");
  return SKV_OK;
}

skv_status launch_attention(const skv_attn_desc* desc, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                            const skv_plan* plan, const void* workspace, float* o_part, float* lse_part,
                            void* stream, const float* k_scales = nullptr, const float* v_scales = nullptr) {
  AttnLaunch a{desc, q, k_pages, v_pages, page_table, seq_lens, workspace, o_part, lse_part,
               (int)plan->tasks.size(), plan->tasks_off, (hipStream_t)stream, plan->max_ntok,
               k_scales, v_scales};
  hipError_t e;
  switch (pick_variant(*desc)) {
    case Variant::GqaValu: e = launch_gqa_valu(a); break;
    case Variant::GqaMfma:
    case Variant::GqaMfmaG8: e = launch_gqa_mfma(a); break;
    default: e = launch_mla_mfma(a); break;
  }
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "attention kernel launch: %s", hipGetErrorString(e));
  return SKV_OK;
}

MergeLaunch merge_launch(const skv_attn_desc* desc, const skv_plan* plan, const void* workspace,
                         const float* o_part, const float* lse_part, int32_t n_ext, const float* o_ext,
                         const float* lse_ext, void* o_out, int32_t out_dtype, float* lse_out, void* stream) {
  int64_t tq = 0;
  for (int64_t n : plan->pb.q_lens) tq += n;
  int max_splits = 1;
  for (const auto& r : plan->ranges) max_splits = std::max(max_splits, (int)r.size());
  return MergeLaunch{workspace, o_part, lse_part, n_ext, o_ext, lse_ext, o_out, out_dtype == SKV_BF16, lse_out,
                     desc->head_dim_v, tq * desc->num_q_heads, (int)plan->units.size(), plan->reqs_off,
                     plan->units_off, (hipStream_t)stream, max_splits + n_ext, plan->run};
}

skv_status launch_merge_for(const skv_attn_desc* desc, const skv_plan* plan, const void* workspace,
                            const float* o_part, const float* lse_part, int32_t n_ext, const float* o_ext,
                            const float* lse_ext, void* o_out, int32_t out_dtype, float* lse_out,
                            void* stream) {
  const MergeLaunch m = merge_launch(desc, plan, workspace, o_part, lse_part, n_ext, o_ext, lse_ext, o_out,
                                     out_dtype, lse_out, stream);
  hipError_t e = launch_merge(m);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return SKV_OK;
}

}  // namespace

namespace skv {

ScratchLayout scratch_layout(const skv_plan* pl) {
  ScratchLayout s;
  const int64_t rows = pl->state_row_offset.back();
  s.counters_off = 0;
  s.o_off = align256(kFusedArgsBytes +
                     sizeof(int32_t) * kFusedCounterLine * (kFusedCounterHead + (size_t)pl->desc.batch));
  s.lse_off = s.o_off + align256((size_t)rows * pl->desc.head_dim_v * sizeof(float));
  s.total = s.lse_off + align256((size_t)rows * sizeof(float));
  return s;
}

skv_status decode_attn_impl(const skv_attn_desc* desc, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                            const skv_plan* plan, const void* workspace, void* scratch,
                            size_t scratch_bytes, int32_t n_ext, const float* o_ext, const float* lse_ext,
                            void* o_out, int32_t out_dtype, float* lse_out, void* stream,
                            const float* k_scales, const float* v_scales) {
  skv_status st = check_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, k_scales,
                                  v_scales);
  if (st) return st;
  if ((st = check_merge(desc, plan, workspace, n_ext, o_ext, lse_ext, o_out, out_dtype))) return st;
  if (desc->dtype == SKV_FP8_E4M3 && plan->prm.overlap_reduction)
    return fail(SKV_ERR_UNSUPPORTED, "FP8 KV runs the two launches: build its plan with overlap_reduction = 0");
  if (!scratch) return fail(SKV_ERR_INVALID_ARG, "scratch is NULL");
  const ScratchLayout lay = scratch_layout(plan);
  if (scratch_bytes < lay.total)
    return fail(SKV_ERR_NO_MEMORY, "scratch holds %zu bytes, the plan needs %zu", scratch_bytes, lay.total);
  uint8_t* base = static_cast<uint8_t*>(scratch);
  float* o_part = reinterpret_cast<float*>(base + lay.o_off);
  float* lse_part = reinterpret_cast<float*>(base + lay.lse_off);
  if (!plan->prm.overlap_reduction) {
    // the plan assumes the merge runs after attention: two launches
    st = launch_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, o_part,
                          lse_part, stream, k_scales, v_scales);
    if (st) return st;
    return launch_merge_for(desc, plan, workspace, o_part, lse_part, n_ext, o_ext, lse_ext, o_out,
                            out_dtype, lse_out, stream);
  }
  // the plan assumes the pages' fused engine: attention and merge in one
  // launch; the setup kernel writes the merge's arguments and clears the
  // counters in the scratch's counters block
  const MergeLaunch m = merge_launch(desc, plan, workspace, o_part, lse_part, n_ext, o_ext, lse_ext, o_out,
                                     out_dtype, lse_out, stream);
  uint8_t* block = base + lay.counters_off;
  hipError_t e = launch_fused_setup(block, m, desc->batch, (int)plan->tasks.size(), (hipStream_t)stream);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "fused setup kernel launch: %s", hipGetErrorString(e));
  AttnLaunch a{desc, q, k_pages, v_pages, page_table, seq_lens, workspace, o_part, lse_part,
               (int)plan->tasks.size(), plan->tasks_off, (hipStream_t)stream, plan->max_ntok};
  const FusedLaunch f{block};
  switch (pick_variant(*desc)) {
    case Variant::GqaValu: e = launch_gqa_valu_fused(a, f); break;
    case Variant::GqaMfma:
    case Variant::GqaMfmaG8: e = launch_gqa_mfma_fused(a, f); break;
    default: e = launch_mla_mfma_fused(a, f); break;
  }
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "fused attention kernel launch: %s", hipGetErrorString(e));
  return SKV_OK;
}

}  // namespace skv

extern "C" {

skv_status skv_decode_attn_partial(const skv_attn_desc* desc, const void* q, const void* k_pages,
                                   const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                                   const skv_plan* plan, const void* workspace, float* o_part,
                                   float* lse_part, void* stream) {
  skv_status st = check_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace);
  if (st) return st;
  if (!o_part || !lse_part) return fail(SKV_ERR_INVALID_ARG, "a device pointer is NULL");
  return launch_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, o_part,
                          lse_part, stream);
}

skv_status skv_decode_attn_partial_fp8(const skv_attn_desc* desc, const void* q, const void* k_pages,
                                       const void* v_pages, const float* k_scales, const float* v_scales,
                                       const int32_t* page_table, const int32_t* seq_lens,
                                       const skv_plan* plan, const void* workspace, float* o_part,
                                       float* lse_part, void* stream) {
  if (desc && desc->dtype != SKV_FP8_E4M3)
    return fail(SKV_ERR_INVALID_ARG, "skv_decode_attn_partial_fp8 needs desc->dtype = SKV_FP8_E4M3");
  skv_status st = check_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace,
                                  k_scales, v_scales);
  if (st) return st;
  if (!o_part || !lse_part) return fail(SKV_ERR_INVALID_ARG, "a device pointer is NULL");
  return launch_attention(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, o_part,
                          lse_part, stream, k_scales, v_scales);
}

skv_status skv_merge_states(const skv_attn_desc* desc, const skv_plan* plan, const void* workspace,
                            const float* o_part, const float* lse_part, int32_t n_ext, const float* o_ext,
                            const float* lse_ext, void* o_out, int32_t out_dtype, float* lse_out,
                            void* stream) {
  skv_status st = check_merge(desc, plan, workspace, n_ext, o_ext, lse_ext, o_out, out_dtype);
  if (st) return st;
  if (!o_part || !lse_part) return fail(SKV_ERR_INVALID_ARG, "a device pointer is NULL");
  return launch_merge_for(desc, plan, workspace, o_part, lse_part, n_ext, o_ext, lse_ext, o_out, out_dtype,
                          lse_out, stream);
}

size_t skv_decode_attn_scratch_bytes(const skv_plan* plan) {
  return plan ? scratch_layout(plan).total : 0;
}

skv_status skv_decode_attn(const skv_attn_desc* desc, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                           const skv_plan* plan, const void* workspace, void* scratch,
                           size_t scratch_bytes, int32_t n_ext, const float* o_ext, const float* lse_ext,
                           void* o_out, int32_t out_dtype, float* lse_out, void* stream) {
  return decode_attn_impl(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, scratch,
                          scratch_bytes, n_ext, o_ext, lse_ext, o_out, out_dtype, lse_out, stream);
}

skv_status skv_decode_attn_fp8(const skv_attn_desc* desc, const void* q, const void* k_pages,
                               const void* v_pages, const float* k_scales, const float* v_scales,
                               const int32_t* page_table, const int32_t* seq_lens, const skv_plan* plan,
                               const void* workspace, void* scratch, size_t scratch_bytes, int32_t n_ext,
                               const float* o_ext, const float* lse_ext, void* o_out, int32_t out_dtype,
                               float* lse_out, void* stream) {
  if (desc && desc->dtype != SKV_FP8_E4M3)
    return fail(SKV_ERR_INVALID_ARG, "skv_decode_attn_fp8 needs desc->dtype = SKV_FP8_E4M3");
  return decode_attn_impl(desc, q, k_pages, v_pages, page_table, seq_lens, plan, workspace, scratch,
                          scratch_bytes, n_ext, o_ext, lse_ext, o_out, out_dtype, lse_out, stream, k_scales,
                          v_scales);
}

skv_status skv_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks,
                              void* stream) {
  if (!buf || !out) return fail(SKV_ERR_INVALID_ARG, "buf or out is NULL");
  if ((uintptr_t)buf % 16 != 0) return fail(SKV_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  if (bytes <= 0 || bytes % 16 != 0) return fail(SKV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (blocks < 1 || blocks > 65536) return fail(SKV_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
  hipError_t e = launch_hbm_probe(buf, bytes, out, blocks, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return SKV_OK;
}

skv_status skv_mfma_probe(const void* buf, int64_t bytes, int32_t passes, uint32_t* out, int32_t blocks,
                          int32_t waves, int32_t mfma_waves, int32_t iters, void* stream) {
  if (!out) return fail(SKV_ERR_INVALID_ARG, "out is NULL");
  if (blocks < 1 || blocks > 65536) return fail(SKV_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
  if (waves < 1 || waves > 8) return fail(SKV_ERR_INVALID_ARG, "waves must be in [1, 8]");
  if (mfma_waves < 0 || mfma_waves > waves) return fail(SKV_ERR_INVALID_ARG, "mfma_waves must be in [0, waves]");
  if (iters < 0 || iters > (1 << 24)) return fail(SKV_ERR_INVALID_ARG, "iters must be in [0, 2^24]");
  if (mfma_waves < waves) {   // streaming waves read the buffer
    if (!buf) return fail(SKV_ERR_INVALID_ARG, "buf is NULL but the launch has streaming waves");
    if ((uintptr_t)buf % 16 != 0) return fail(SKV_ERR_INVALID_ARG, "buf must be 16-byte aligned");
    if (bytes <= 0 || bytes % 16 != 0) return fail(SKV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (passes < 0 || passes > 1024) return fail(SKV_ERR_INVALID_ARG, "passes must be in [0, 1024]");
  }
  hipError_t e = launch_mfma_probe(buf, mfma_waves < waves ? bytes : 0, mfma_waves < waves ? passes : 0, blocks,
                                   waves, mfma_waves, iters, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return SKV_OK;
}

skv_status skv_read_error_flag(const void* workspace, int32_t* flag, void* stream) {
  if (!workspace || !flag) return fail(SKV_ERR_INVALID_ARG, "workspace or flag is NULL");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpy(flag, workspace, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SKV_ERR_HIP, "reading the error flag: %s", hipGetErrorString(e));
  return SKV_OK;
}

const char* skv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace skv {
VariantShape variant_shape(Variant v) {
  switch (v) {
    case Variant::GqaValu: return {8, 16};
    case Variant::GqaMfma: return {2, 16};
    case Variant::GqaMfmaG8: return {4, 16};
    default: return {1, 16};
  }
}

// Critical-wave parameters for each kernel on MI355X, from the table the
// calibration tool writes (split_kv_partial_amd/calibrate.py): the model of
// LiquidCP section 5.2 fitted to timed plans per kernel as in appendix A.2,
// then validated on the planner's own plans for the workloads the kernel
// serves (the model's identical slots at one rate cannot see how tasks spread
// over CUs, so the fit of least error is not always the fastest). The last
// field turns on the proportional candidates by default: on the MLA 64-request
// DeepSeek shape the one-task-per-slot proportional plan the model prefers ran
// 0.6-3.6% faster than the search result in alternating runs; on the GQA
// 32-request shape the model's one-wave proportional plan ran 1% slower than
// the two-wave search result, so GQA keeps the pages' candidates.
Calibration calibration(Variant v) {
  // the table written by the calibration tool (split_kv_partial_amd/calibrate.py)
#define CAL(V, rho, delta_attn, delta_red, gamma, tile_time_us, balanced) \
  if (v == Variant::V) return {rho, delta_attn, delta_red, gamma, tile_time_us, balanced};
#include "calibration_mi355x.inc"
#undef CAL
  return {1.0, 2.0, 1.0, 0.47, 1.0, 0};   // not reached: every variant has a row
}
}  // namespace skv
