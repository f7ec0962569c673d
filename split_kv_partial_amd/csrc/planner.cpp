// Critical-wave split planner (LiquidCP, section 5.2 "Critical-wave KV
// splitting", Equations 5-6, "Plan selection", "Task ordering"; appendix A.2
// "Split planning").
//
// Model: time unit = one KV tile per attention slot with all K slots busy. With
// k slots running attention every running task advances at 1 / tau(k),
// tau(k) = max(rho, k / K). A task costs c_attn = n_t + delta_attn; a reduction
// unit costs c_red = delta_red + gamma * v_u * s_u. Tasks go in queue order to
// the lowest-index free slot; reductions are claimed in queue order by the
// earliest-free warp and start when their request's attention has finished.
//
// The simulation keeps a "work clock" w = integral of 1/tau(k) dt: a task that
// starts at work w0 finishes when the clock reaches w0 + c, so simultaneous
// finishes stay exactly simultaneous. Doubles are combined in a fixed order
// (this file is built without floating-point contraction) so the scores are
// reproducible bit for bit.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <map>
#include <numeric>
#include <tuple>
#include <vector>

#include "internal.hpp"
#include "sim_pool.hpp"

namespace skv {

int64_t n_tiles(int64_t L, int T) { return (L + T - 1) / T; }

// n tiles in s parts: the first n mod s parts are one tile longer (Figure 8
// splits 176 tiles in three as 59, 59, 58).
static std::vector<std::pair<int64_t, int64_t>> split_tiles(int64_t n, int s) {
  std::vector<std::pair<int64_t, int64_t>> out;
  out.reserve(s);
  int64_t q = n / s, rem = n % s, start = 0;
  for (int r = 0; r < s; ++r) {
    int64_t size = q + (r < rem ? 1 : 0);
    out.emplace_back(start, start + size);
    start += size;
  }
  return out;
}

std::vector<std::pair<int64_t, int64_t>> split_ranges(int64_t L, int s, int T) {
  auto t = split_tiles(n_tiles(L, T), s);
  for (auto& p : t) {
    p.first *= T;
    p.second = std::min<int64_t>(p.second * T, L);
  }
  return t;
}

static bool is_decode(int64_t n) { return n <= 16; }

// Query tiles of a request with n query tokens: qt consecutive tokens each (the
// last may hold fewer). One attention task per (query tile, KV head, split);
// its KV tiles are those its last token sees.
static int64_t num_qtiles(int64_t n, int qt) { return (n + qt - 1) / qt; }
static int64_t qtile_last(int64_t n, int qt, int64_t k) { return std::min<int64_t>(n, (k + 1) * qt) - 1; }

// Tasks of a plan in queue order: FIFO enumerates (request, query tile, KV head,
// split); split decode-only plans are reordered longest-first (stable); batches
// with chunk requests (more than 16 query tokens) put those requests' tasks first.
void build_tasks(const Problem& pb, const ModelParams& prm,
                 const std::vector<std::vector<std::pair<int64_t, int64_t>>>& ranges,
                 std::vector<TaskDesc>& out, std::vector<double>* costs) {
  const int T = prm.tile_tokens;
  const int B = (int)pb.seq_lens.size();
  std::vector<TaskDesc> fifo;
  std::vector<double> c;
  std::vector<int64_t> qoff(B + 1, 0);
  for (int b = 0; b < B; ++b) qoff[b + 1] = qoff[b] + pb.q_lens[b];
  bool any_split = false, decode_only = true;
  for (int b = 0; b < B; ++b) {
    any_split |= ranges[b].size() > 1;
    decode_only &= is_decode(pb.q_lens[b]);
  }
  const int qt = pb.query_tile;
  for (int b = 0; b < B; ++b) {
    const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
    for (int64_t qi = 0; qi < num_qtiles(n, qt); ++qi) {
      const int64_t vis = pb.causal ? L - n + qtile_last(n, qt, qi) + 1 : L;
      const int64_t vis_t = n_tiles(vis, T);
      for (int g = 0; g < pb.num_kv_heads; ++g) {
        for (int r = 0; r < (int)ranges[b].size(); ++r) {
          const int64_t lo = ranges[b][r].first, hi = ranges[b][r].second;
          const int64_t lo_t = lo / T, hi_t = n_tiles(hi, T);
          const int64_t nt = std::max<int64_t>(0, std::min(hi_t, vis_t) - lo_t);
          TaskDesc t{b, g, (int32_t)qi, r, (int32_t)lo, (int32_t)hi,
                     (int32_t)(qoff[b] + qi * qt), 0};
          fifo.push_back(t);
          c.push_back((double)nt + prm.delta_attn);
        }
      }
    }
  }
  std::vector<size_t> idx(fifo.size());
  std::iota(idx.begin(), idx.end(), 0);
  if (decode_only && any_split) {
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return c[a] > c[b]; });
  } else if (!decode_only) {
    std::stable_partition(idx.begin(), idx.end(),
                          [&](size_t a) { return !is_decode(pb.q_lens[fifo[a].b]); });
  }
  out.clear();
  out.reserve(fifo.size());
  if (costs) {
    costs->clear();
    costs->reserve(fifo.size());
  }
  for (size_t i : idx) {
    out.push_back(fifo[i]);
    if (costs) costs->push_back(c[i]);
  }
}

// Rows per reduction unit: the largest run in {1, h, 2h, 4h, min(8h, 32)} that
// leaves at least 0.8 x (K x warps) units (appendix A.2).
int reduction_run(const Problem& pb, const ModelParams& prm) {
  const int64_t h = pb.rows_per_token;
  const double warps = (double)prm.slots * (double)prm.warps_per_slot;
  const int64_t cand[5] = {1, h, 2 * h, 4 * h, std::min<int64_t>(8 * h, 32)};
  int64_t best = 1;
  for (int64_t run : cand) {
    int64_t units = 0;
    for (int64_t n : pb.q_lens) units += (n * h + run - 1) / run;
    if ((double)units >= 0.8 * warps && run > best) best = run;
  }
  return (int)best;
}

namespace {

// Slots are identical and warps are identical, so the simulation tracks
// multisets of times rather than which slot or warp holds what: which of several
// equally early slots takes the next task changes no time in the model. Tasks
// that start together with equal costs finish together and are kept as one
// group. Every time is computed with the same double operations in the same
// order as a per-task, per-slot event simulation, so the results are equal bit
// for bit.
struct Group {
  double fw;     // work-clock value at which the group's tasks finish
  int64_t n;     // tasks in the group
  bool operator>(const Group& o) const { return fw > o.fw; }
};

// A run of consecutive queued tasks of one request with equal cost. Such tasks
// are interchangeable in the model (same cost, same request), so the queue is
// kept as runs rather than single tasks.
struct QEntry {
  double cost;
  int32_t req;
  int64_t count;
};

// A queue is a sequence of segments of runs (one segment per request for the
// FIFO orders, one merged segment for the longest-first order).
struct Seg {
  const QEntry* p;
  size_t n;
};

// Request b's tasks with s splits in FIFO order (query tile, KV head, split),
// consecutive equal costs merged.
void request_fifo(const Problem& pb, const ModelParams& prm, int b, int s, std::vector<QEntry>& out) {
  out.clear();
  const int T = prm.tile_tokens;
  const int qt = pb.query_tile;
  const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
  const int64_t total = n_tiles(L, T);
  for (int64_t qi = 0; qi < num_qtiles(n, qt); ++qi) {
    const int64_t vis = pb.causal ? L - n + qtile_last(n, qt, qi) + 1 : L;
    const int64_t vis_t = n_tiles(vis, T);
    for (int g = 0; g < pb.num_kv_heads; ++g) {
      // the same tile split as split_ranges: the first total mod s parts are
      // one tile longer
      int64_t lo_t = 0;
      for (int r = 0; r < s; ++r) {
        const int64_t len = total / s + (r < total % s ? 1 : 0);
        const int64_t hi_t = lo_t + len;
        const int64_t nt = std::max<int64_t>(0, std::min(hi_t, vis_t) - lo_t);
        const double c = (double)nt + prm.delta_attn;
        if (!out.empty() && out.back().cost == c)
          ++out.back().count;
        else
          out.push_back({c, b, 1});
        lo_t = hi_t;
      }
    }
  }
}

// The same tasks longest first: one run per distinct cost, costs descending.
void request_sorted(const std::vector<QEntry>& fifo, std::vector<QEntry>& out) {
  out.assign(fifo.begin(), fifo.end());
  std::sort(out.begin(), out.end(), [](const QEntry& x, const QEntry& y) { return x.cost > y.cost; });
  size_t w = 0;
  for (size_t i = 0; i < out.size(); ++i) {
    if (w > 0 && out[w - 1].cost == out[i].cost)
      out[w - 1].count += out[i].count;
    else
      out[w++] = out[i];
  }
  out.resize(w);
}

// Longest-first queue order of the whole batch: costs descending, and among
// equal costs the earlier request first (a stable sort of the FIFO queue).
bool lpt_before(const QEntry& x, const QEntry& y) {
  return x.cost > y.cost || (x.cost == y.cost && x.req < y.req);
}

// Which order build_tasks uses for this plan.
enum class QOrder { Fifo, Lpt, ChunkFirst };
QOrder queue_order(const Problem& pb, const std::vector<int>& splits) {
  bool any_split = false, decode_only = true;
  for (size_t b = 0; b < splits.size(); ++b) {
    any_split |= splits[b] > 1;
    decode_only &= is_decode(pb.q_lens[b]);
  }
  if (decode_only && any_split) return QOrder::Lpt;
  return decode_only ? QOrder::Fifo : QOrder::ChunkFirst;
}

struct SimScratch {
  std::vector<Group> step_groups;
  std::vector<double> done_fw, ev_fw, ev_t, done, sufmax;
  std::vector<size_t> seg_base;
  std::vector<Group> heap;
  std::vector<std::pair<double, int64_t>> warps;   // min-heap of (free time, warps)
  std::vector<QEntry> tmp;
  std::vector<std::vector<QEntry>> per_req;
  std::vector<Seg> segs;
};

struct SimResult {
  double score = 0, t_attn = 0;
  int64_t n_tasks = 0;
  bool cut = false;   // abandoned: its score exceeds the cutoff
};

bool warp_later(const std::pair<double, int64_t>& x, const std::pair<double, int64_t>& y) {
  return x.first > y.first;
}

// State of a run just before one of its task-start steps, from which a run
// over a queue that agrees with it up to the entries that step reads can
// continue (the steps before it cannot tell the two queues apart).
struct Snapshot {
  double t = 0, vw = 0;
  int64_t running = 0, started = 0;   // tasks running / started before the step
  int64_t free_slots = 0;             // slots the step fills
  size_t si = 0, ei = 0;              // queue position (segment, run)
  int64_t off = 0;                    // tasks of that run already started
  size_t n_ev = 0;                    // events before the step, its own included
  std::vector<Group> heap;
  std::vector<double> done_fw;
};

// A recording run: its events, and for each resume threshold (a global run
// index, ascending) the state before the first step that reads that run.
struct Recording {
  std::vector<int64_t> thresholds;
  std::vector<size_t> snap_of;        // per threshold, index into snaps
  std::vector<Snapshot> snaps;
  std::vector<double> ev_fw, ev_t;
};

// The model run over a queue given as segments of runs. tail (optional)
// receives the requests whose attention ends at the attention completion.
// With `from`, the run continues from a snapshot of the recording `base`; with
// `rec` (non-overlapped model only), it records snapshots for rec->thresholds.
// With `cutoff` (non-overlapped model only), the run is abandoned (cut) as
// soon as a lower bound on its score exceeds *cutoff (a score that some other
// run has reached): the time so far; plus the remaining attention time, at
// least the remaining task cost (unstarted, and the rest of the running ones)
// over K, since attention advances by at most K tile units per time unit, and
// at least rho times the largest remaining cost of one task (an unstarted one,
// or the rest of the last running one), since a task advances by at most
// 1 / rho per time unit; plus the reduction phase's lower bound (the largest
// unit cost, and the summed unit cost over K x W warps: every unit starts
// after attention).
SimResult simulate_queue(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits,
                         const Seg* segs, size_t nseg, SimScratch& sc, std::vector<int>* tail,
                         const Snapshot* from = nullptr, const Recording* base = nullptr,
                         Recording* rec = nullptr, int run_hint = 0,
                         const std::atomic<double>* cutoff = nullptr) {
  const int B = (int)pb.seq_lens.size();
  const int64_t K = prm.slots;
  int64_t nt = 0;
  for (size_t i = 0; i < nseg; ++i)
    for (size_t j = 0; j < segs[i].n; ++j) nt += segs[i].p[j].count;
  const int run = run_hint > 0 ? run_hint : reduction_run(pb, prm);
  // Per-request attention ends are needed for the overlapped model's
  // reductions and for `tail`. Otherwise every reduction starts at the
  // attention completion or later (the warps are released there), whatever
  // its request's end, so the events need not be kept.
  const bool track = prm.overlap_reduction || tail != nullptr;
  double w_left = 0, red_lb = 0;   // unstarted task cost; reduction-phase bound
  double w_end = 0, fw_max = 0;    // running groups: sum of count x finish, latest finish
  std::vector<size_t>& seg_base = sc.seg_base;
  std::vector<double>& sufmax = sc.sufmax;   // largest cost from each queue position on
  if (cutoff) {
    seg_base.assign(nseg + 1, 0);
    for (size_t i = 0; i < nseg; ++i) seg_base[i + 1] = seg_base[i] + segs[i].n;
    sufmax.assign(seg_base[nseg] + 1, 0.0);
    for (size_t i = nseg; i-- > 0;)
      for (size_t j = segs[i].n; j-- > 0;)
        sufmax[seg_base[i] + j] = std::max(sufmax[seg_base[i] + j + 1], segs[i].p[j].cost);
    const size_t s0 = from ? from->si : 0, e0 = from ? from->ei : 0;
    for (size_t i = s0; i < nseg; ++i)
      for (size_t j = i == s0 ? e0 : 0; j < segs[i].n; ++j)
        w_left += segs[i].p[j].cost * (double)segs[i].p[j].count;
    if (from && s0 < nseg && e0 < segs[s0].n) w_left -= segs[s0].p[e0].cost * (double)from->off;
    if (from)
      for (const Group& gr : from->heap) {
        w_end += gr.fw * (double)gr.n;
        fw_max = std::max(fw_max, gr.fw);
      }
    double rmax = 0, rsum = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t rows = pb.q_lens[b] * (int64_t)pb.rows_per_token;
      const double s_u = (double)(splits[b] + pb.n_ext);
      const int64_t full = rows / run, rem = rows % run;
      rsum += (double)full * (prm.delta_red + prm.gamma * (double)run * s_u);
      if (rem > 0) rsum += prm.delta_red + prm.gamma * (double)rem * s_u;
      rmax = std::max(rmax, prm.delta_red + prm.gamma * (double)(rows >= run ? run : rows) * s_u);
    }
    red_lb = std::max(rmax, rsum / ((double)K * (double)prm.warps_per_slot));
  }

  // ---- attention phase ----
  sc.ev_fw.clear();
  sc.ev_t.clear();
  std::map<double, int64_t> release;  // slot release times (overlapped reductions only)
  auto heap_push = [&](double fw, int64_t n) {
    sc.heap.push_back({fw, n});
    std::push_heap(sc.heap.begin(), sc.heap.end(), std::greater<Group>());
    if (cutoff) {
      w_end += fw * (double)n;
      fw_max = std::max(fw_max, fw);
    }
  };
  double t = 0.0, vw = 0.0;
  int64_t running = 0, started_total = 0;
  size_t si = 0, ei = 0;   // queue position: segment, run
  int64_t off = 0;         // tasks of the current run already started
  size_t n_prefix = 0;     // events taken from `base`
  if (from) {
    sc.done_fw.assign(from->done_fw.begin(), from->done_fw.end());
    sc.heap.assign(from->heap.begin(), from->heap.end());
    t = from->t;
    vw = from->vw;
    running = from->running;
    started_total = from->started;
    si = from->si;
    ei = from->ei;
    off = from->off;
    n_prefix = from->n_ev;
  } else {
    sc.done_fw.assign(B, 0.0);
    sc.heap.clear();
  }
  std::vector<size_t> seg_start;
  if (rec) {
    seg_start.resize(nseg + 1, 0);
    for (size_t i = 0; i < nseg; ++i) seg_start[i + 1] = seg_start[i] + segs[i].n;
    rec->snap_of.assign(rec->thresholds.size(), 0);
    rec->snaps.clear();
  }
  size_t next_thr = 0;
  int64_t max_read = -1;
  auto skip_empty = [&] {
    while (si < nseg && ei >= segs[si].n) {
      ++si;
      ei = 0;
    }
  };
  skip_empty();
  auto entry = [&]() -> const QEntry& {
    if (rec) max_read = std::max<int64_t>(max_read, (int64_t)(seg_start[si] + ei));
    return segs[si].p[ei];
  };
  // start up to free_slots queued tasks at work clock vw, one group per cost
  // (stretches of equal cost started in the same step finish together, and
  // the event loop takes every group of one finish time at once, so they are
  // one group); returns how many started
  auto& step_groups = sc.step_groups;
  auto start_tasks = [&](int64_t free_slots) {
    int64_t started = 0;
    step_groups.clear();
    while (started < free_slots && started_total < nt) {
      const double c = entry().cost;
      const double fw = vw + c;
      const int64_t lim = free_slots - started;
      int64_t taken = 0;
      while (taken < lim && si < nseg && entry().cost == c) {
        const QEntry& e = segs[si].p[ei];
        const int64_t k = std::min(e.count - off, lim - taken);
        if (fw > sc.done_fw[e.req]) sc.done_fw[e.req] = fw;
        taken += k;
        off += k;
        if (off == e.count) {
          off = 0;
          ++ei;
          skip_empty();
        }
      }
      size_t g = 0;
      while (g < step_groups.size() && step_groups[g].fw != fw) ++g;
      if (g < step_groups.size())
        step_groups[g].n += taken;
      else if (step_groups.size() < 16)
        step_groups.push_back({fw, taken});
      else
        heap_push(fw, taken);
      if (cutoff) w_left -= c * (double)taken;
      started += taken;
      started_total += taken;
    }
    for (const Group& gr : step_groups) heap_push(gr.fw, gr.n);
    running += started;
    return started;
  };
  // a task-start step, recorded when a pending threshold is within its reach
  // (a step filling m slots reads at most m + 1 runs)
  auto step = [&](int64_t free_slots) {
    if (!rec || next_thr >= rec->thresholds.size()) return start_tasks(free_slots);
    const int64_t pos = si < nseg ? (int64_t)(seg_start[si] + ei) : (int64_t)seg_start[nseg];
    const bool reach = rec->thresholds[next_thr] <= pos + free_slots;
    if (reach) {
      Snapshot sn;
      sn.t = t;
      sn.vw = vw;
      sn.running = running;
      sn.started = started_total;
      sn.free_slots = free_slots;
      sn.si = si;
      sn.ei = ei;
      sn.off = off;
      sn.n_ev = sc.ev_fw.size();
      sn.heap = sc.heap;
      sn.done_fw = sc.done_fw;
      rec->snaps.push_back(std::move(sn));
    }
    const int64_t r = start_tasks(free_slots);
    if (reach) {
      bool used = false;
      while (next_thr < rec->thresholds.size() && rec->thresholds[next_thr] <= max_read) {
        rec->snap_of[next_thr++] = rec->snaps.size() - 1;
        used = true;
      }
      if (!used) rec->snaps.pop_back();
    }
    return r;
  };
  if (from) {
    step(from->free_slots);
  } else {
    step(K);
    if (prm.overlap_reduction && K > nt) release[0.0] += (K - nt) * prm.warps_per_slot;
  }
  uint32_t n_events = 0;
  while (!sc.heap.empty()) {
    if (cutoff && (++n_events & 15) == 0) {
      const double bst = cutoff->load(std::memory_order_relaxed);
      const double c_next = si < nseg ? sufmax[seg_base[si] + ei] : 0.0;
      const double rest = std::max((w_left + (w_end - (double)running * vw)) / (double)K,
                                   prm.rho * std::max(c_next, fw_max - vw));
      if (t + rest + red_lb > bst + 1e-9 * std::fabs(bst)) {
        SimResult cut;
        cut.score = cut.t_attn = INFINITY;
        cut.n_tasks = nt;
        cut.cut = true;
        return cut;
      }
    }
    const double tau = std::max(prm.rho, (double)running / (double)K);
    const double fw = sc.heap.front().fw;
    t = t + (fw - vw) * tau;
    vw = fw;
    int64_t m = 0;
    while (!sc.heap.empty() && sc.heap.front().fw == fw) {
      m += sc.heap.front().n;
      if (cutoff) w_end -= fw * (double)sc.heap.front().n;
      std::pop_heap(sc.heap.begin(), sc.heap.end(), std::greater<Group>());
      sc.heap.pop_back();
    }
    running -= m;
    if (track) {
      sc.ev_fw.push_back(fw);
      sc.ev_t.push_back(t);
    }
    const int64_t started = step(m);
    if (prm.overlap_reduction && m > started) release[t] += (m - started) * prm.warps_per_slot;
  }
  const double t_attn = t;
  // a request's attention ends at the event of its latest-finishing task (the
  // events are the recording's first n_prefix, then this run's own)
  sc.done.assign(B, 0.0);
  const double* pfw = base ? base->ev_fw.data() : nullptr;
  const double* pt = base ? base->ev_t.data() : nullptr;
  for (int b = 0; track && b < B; ++b) {
    const double f = sc.done_fw[b];
    if (f == 0.0) continue;  // no task started (cannot happen: every request has one)
    if (n_prefix > 0 && f <= pfw[n_prefix - 1]) {
      sc.done[b] = pt[std::lower_bound(pfw, pfw + n_prefix, f) - pfw];
    } else {
      const auto it = std::lower_bound(sc.ev_fw.begin(), sc.ev_fw.end(), f);
      sc.done[b] = sc.ev_t[it - sc.ev_fw.begin()];
    }
  }
  if (rec) {
    rec->ev_fw.assign(sc.ev_fw.begin(), sc.ev_fw.end());
    rec->ev_t.assign(sc.ev_t.begin(), sc.ev_t.end());
  }

  // ---- reduction phase: units in request order, each on the earliest-free warp ----
  // (a heap of (free time, count) groups; equal times need not be merged, since
  // every unit still starts at the earliest free time)
  const int64_t nwarps = K * prm.warps_per_slot;
  auto& wh = sc.warps;
  wh.clear();
  if (prm.overlap_reduction) {
    for (const auto& kv : release) wh.push_back(kv);
    std::make_heap(wh.begin(), wh.end(), warp_later);
  } else {
    wh.push_back({t_attn, nwarps});
  }
  double score = t_attn;
  auto assign = [&](int64_t k, double c, double d) {
    while (k > 0) {
      const double a = wh.front().first;
      const int64_t avail = wh.front().second;
      const double st = a > d ? a : d;
      const double end = st + c;
      const int64_t j = std::min(k, avail);
      if (j == avail) {
        std::pop_heap(wh.begin(), wh.end(), warp_later);
        wh.pop_back();
      } else {
        wh.front().second -= j;
      }
      wh.push_back({end, j});
      std::push_heap(wh.begin(), wh.end(), warp_later);
      if (end > score) score = end;
      k -= j;
    }
  };
  for (int b = 0; b < B; ++b) {
    const int64_t rows = pb.q_lens[b] * (int64_t)pb.rows_per_token;
    const int64_t s_u = splits[b] + pb.n_ext;
    const int64_t full = rows / run, rem = rows % run;
    if (full > 0) assign(full, prm.delta_red + prm.gamma * (double)run * (double)s_u, sc.done[b]);
    if (rem > 0) assign(1, prm.delta_red + prm.gamma * (double)rem * (double)s_u, sc.done[b]);
  }
  if (tail) {
    tail->clear();
    for (int b = 0; b < B; ++b)
      if (sc.done[b] == t_attn) tail->push_back(b);
  }
  return {score, t_attn, nt};
}

// Segments of a plan's queue built from scratch.
void build_queue(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits,
                 SimScratch& sc) {
  const int B = (int)pb.seq_lens.size();
  const QOrder ord = queue_order(pb, splits);
  sc.per_req.resize(B);
  for (int b = 0; b < B; ++b) request_fifo(pb, prm, b, splits[b], sc.per_req[b]);
  sc.segs.clear();
  if (ord == QOrder::Lpt) {
    sc.tmp.clear();
    std::vector<QEntry> srt;
    for (int b = 0; b < B; ++b) {
      request_sorted(sc.per_req[b], srt);
      sc.tmp.insert(sc.tmp.end(), srt.begin(), srt.end());
    }
    std::stable_sort(sc.tmp.begin(), sc.tmp.end(), lpt_before);
    sc.segs.push_back({sc.tmp.data(), sc.tmp.size()});
    return;
  }
  if (ord == QOrder::ChunkFirst)
    for (int b = 0; b < B; ++b)
      if (!is_decode(pb.q_lens[b])) sc.segs.push_back({sc.per_req[b].data(), sc.per_req[b].size()});
  for (int b = 0; b < B; ++b)
    if (ord == QOrder::Fifo || is_decode(pb.q_lens[b]))
      sc.segs.push_back({sc.per_req[b].data(), sc.per_req[b].size()});
}

Evaluation to_eval(const std::vector<int>& splits, const SimResult& r, std::vector<int>&& tail) {
  Evaluation ev;
  ev.splits = splits;
  ev.score = r.score;
  ev.t_attn = r.t_attn;
  ev.n_tasks = r.n_tasks;
  ev.total_splits = std::accumulate(splits.begin(), splits.end(), (int64_t)0);
  ev.tail = std::move(tail);
  return ev;
}

}  // namespace

Evaluation simulate(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits) {
  thread_local SimScratch sc;
  build_queue(pb, prm, splits, sc);
  std::vector<int> tail;
  const SimResult r = simulate_queue(pb, prm, splits, sc.segs.data(), sc.segs.size(), sc, &tail);
  return to_eval(splits, r, std::move(tail));
}

// The same with a cutoff (non-overlapped model): false if the run was cut.
static bool simulate_below(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits,
                           const std::atomic<double>& cutoff, Evaluation& out) {
  thread_local SimScratch sc;
  build_queue(pb, prm, splits, sc);
  const SimResult r = simulate_queue(pb, prm, splits, sc.segs.data(), sc.segs.size(), sc, nullptr, nullptr,
                                     nullptr, nullptr, 0, &cutoff);
  if (r.cut) return false;
  out = to_eval(splits, r, {});
  return true;
}

static bool key_less(const Evaluation& a, const Evaluation& b) {
  return std::tie(a.score, a.t_attn, a.n_tasks, a.total_splits) <
         std::tie(b.score, b.t_attn, b.n_tasks, b.total_splits);
}

static std::vector<int> uniform_plan(const Problem& pb, const ModelParams& prm, int u) {
  const int B = (int)pb.seq_lens.size();
  std::vector<int> out(B);
  for (int b = 0; b < B; ++b)
    out[b] = (int)std::max<int64_t>(
        1, std::min<int64_t>({(int64_t)u, n_tiles(pb.seq_lens[b], prm.tile_tokens), (int64_t)prm.max_splits}));
  return out;
}

static SimPool& sim_pool() {
  static SimPool pool;
  return pool;
}

// vis[b]: request b's visible tiles summed over its query tiles.
static std::vector<int64_t> visible_tiles(const Problem& pb, const ModelParams& prm) {
  std::vector<int64_t> vis(pb.seq_lens.size(), 0);
  for (size_t b = 0; b < vis.size(); ++b) {
    const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
    for (int64_t qi = 0; qi < num_qtiles(n, pb.query_tile); ++qi)
      vis[b] += n_tiles(pb.causal ? L - n + qtile_last(n, pb.query_tile, qi) + 1 : L, prm.tile_tokens);
  }
  return vis;
}

// A lower bound on a plan's score in the non-overlapped model. However many
// slots run, attention advances by at most K tile units per time unit
// (k / tau(k) <= K), so the attention completion is at least the summed task
// cost over K; and a task of cost c runs at least rho c (tau >= rho), so it is
// at least rho times the largest task cost (a request's first split, which
// its last query token sees whole). Every reduction starts after it, on K x W
// warps: the score adds at least the summed unit cost over K x W and the
// largest unit cost. A query token's splits cover its visible tiles once, so
// the task cost sums to heads x visible tiles + delta_attn per task.
static double score_lower_bound(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits,
                                const std::vector<int64_t>& vis, int run) {
  const int T = prm.tile_tokens;
  double w = 0, r = 0, tmax = 0, rmax = 0;
  for (size_t b = 0; b < splits.size(); ++b) {
    const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
    const int qt = pb.query_tile;
    w += (double)pb.num_kv_heads *
         ((double)vis[b] + prm.delta_attn * (double)num_qtiles(n, qt) * (double)splits[b]);
    tmax = std::max(tmax, (double)((n_tiles(L, T) + splits[b] - 1) / splits[b]) + prm.delta_attn);
    const int64_t rows = n * (int64_t)pb.rows_per_token;
    const double s_u = (double)(splits[b] + pb.n_ext);
    const int64_t full = rows / run, rem = rows % run;
    r += (double)full * (prm.delta_red + prm.gamma * (double)run * s_u);
    if (rem > 0) r += prm.delta_red + prm.gamma * (double)rem * s_u;
    rmax = std::max(rmax, prm.delta_red + prm.gamma * (double)(rows >= run ? run : rows) * s_u);
  }
  const double K = (double)prm.slots;
  return std::max(prm.rho * tmax, w / K) + std::max(rmax, r / (K * (double)prm.warps_per_slot));
}

// Stand-in for the pages' FA3-derived reference plan (FA3's heuristic is not
// given): one batch-wide split count, capped per request by its tiles, chosen
// by the model among 1..max_splits (ties: the pages' keys, then the smaller
// count). Counts are simulated on worker threads, lowest score bound first;
// a count whose bound exceeds the best score found so far cannot win and is
// not simulated (non-overlapped model; the margin covers rounding in the
// bound). The pick among simulated counts is sequential.
std::vector<int> reference_plan(const Problem& pb, const ModelParams& prm, Evaluation* ev_out) {
  const int U = prm.max_splits;
  std::vector<Evaluation> evs(U);
  std::vector<char> done(U, 0);
  SimPool& pool = sim_pool();
  if (prm.overlap_reduction) {
    pool.run((size_t)U, [&](size_t i) { evs[i] = simulate(pb, prm, uniform_plan(pb, prm, (int)i + 1)); });
    std::fill(done.begin(), done.end(), 1);
  } else {
    std::vector<double> lb(U);
    std::vector<int> order(U);
    const std::vector<int64_t> vis = visible_tiles(pb, prm);
    const int run = reduction_run(pb, prm);
    for (int u = 1; u <= U; ++u) {
      lb[u - 1] = score_lower_bound(pb, prm, uniform_plan(pb, prm, u), vis, run);
      order[u - 1] = u - 1;
    }
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lb[x] < lb[y]; });
    // items are claimed in bound order; one whose bound exceeds the best score
    // found so far cannot win whenever it is skipped
    std::atomic<double> best{INFINITY};
    pool.run((size_t)U, [&](size_t i) {
      const int u = order[i] + 1;
      const double bst = best.load();
      if (lb[u - 1] > bst + 1e-9 * std::fabs(bst)) return;
      if (!simulate_below(pb, prm, uniform_plan(pb, prm, u), best, evs[u - 1])) return;
      done[u - 1] = 1;
      double cur = best.load();
      while (evs[u - 1].score < cur && !best.compare_exchange_weak(cur, evs[u - 1].score)) {
      }
    });
  }
  int best_u = 0;
  for (int u = 1; u <= U; ++u)
    if (done[u - 1] && (best_u == 0 || key_less(evs[u - 1], evs[best_u - 1]))) best_u = u;
  if (ev_out) *ev_out = evs[best_u - 1];
  return uniform_plan(pb, prm, best_u);
}

// Proportional plan whose attention tasks fit wave_tasks (an addition to the
// pages' candidates): the smallest per-split tile budget t such that request b
// with min(ceil(n_b / t), n_b, max_splits) splits (at least one) gives at most
// wave_tasks tasks in all; empty if even NoSplit has more. The task count does
// not increase with t, so t is found by bisection.
std::vector<int> balanced_plan(const Problem& pb, const ModelParams& prm, int64_t wave_tasks) {
  const int B = (int)pb.seq_lens.size();
  std::vector<int64_t> nt(B), per_split(B);
  int64_t hi = 1;
  for (int b = 0; b < B; ++b) {
    nt[b] = n_tiles(pb.seq_lens[b], prm.tile_tokens);
    per_split[b] = num_qtiles(pb.q_lens[b], pb.query_tile) * (int64_t)pb.num_kv_heads;
    hi = std::max(hi, nt[b]);
  }
  std::vector<int> c(B);
  auto tasks_at = [&](int64_t t) {
    int64_t tasks = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t s = std::max<int64_t>(1, std::min<int64_t>({(nt[b] + t - 1) / t, nt[b], (int64_t)prm.max_splits}));
      c[b] = (int)s;
      tasks += s * per_split[b];
    }
    return tasks;
  };
  if (tasks_at(hi) > wave_tasks) return {};
  int64_t lo = 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (tasks_at(mid) <= wave_tasks) hi = mid;
    else lo = mid + 1;
  }
  tasks_at(lo);
  return c;
}

std::vector<int> split_limits(const Problem& pb, const ModelParams& prm,
                              const std::vector<int>& ref) {
  const int B = (int)pb.seq_lens.size();
  std::vector<int> out(B);
  for (int b = 0; b < B; ++b) {
    const int64_t nt = n_tiles(pb.seq_lens[b], prm.tile_tokens);
    int64_t u = ref[b];
    if (is_decode(pb.q_lens[b]) && nt >= prm.slots) u = std::max<int64_t>(u, 4);
    out[b] = (int)std::max<int64_t>(1, std::min<int64_t>({u, nt, (int64_t)prm.max_splits}));
  }
  return out;
}

namespace {

// Per-request queue runs for the request's current split count and the next
// one, so a search candidate's queue is assembled without rebuilding every
// request's tasks.
struct ReqRuns {
  int s = 0;                                  // split count of fifo[0], sorted[0]
  std::vector<QEntry> fifo[2], sorted[2];     // [0]: s splits, [1]: s + 1
};

void fill_runs(const Problem& pb, const ModelParams& prm, int b, int s, ReqRuns& rr) {
  rr.s = s;
  for (int k = 0; k < 2; ++k) {
    request_fifo(pb, prm, b, s + k, rr.fifo[k]);
    request_sorted(rr.fifo[k], rr.sorted[k]);
  }
}

// Longest-first queue of `base` (the current plan's, merged over requests) with
// the requests marked in `changed` (listed in `clist`, ascending) replaced by
// their runs for one more split.
void merge_lpt(const std::vector<QEntry>& base, const std::vector<ReqRuns>& runs,
               const std::vector<int>& clist, const std::vector<uint8_t>& changed,
               std::vector<QEntry>& added, std::vector<QEntry>& out) {
  added.clear();
  for (int b : clist) added.insert(added.end(), runs[b].sorted[1].begin(), runs[b].sorted[1].end());
  std::stable_sort(added.begin(), added.end(), lpt_before);
  out.clear();
  size_t j = 0;
  for (const QEntry& e : base) {
    if (changed[e.req]) continue;
    while (j < added.size() && lpt_before(added[j], e)) out.push_back(added[j++]);
    out.push_back(e);
  }
  while (j < added.size()) out.push_back(added[j++]);
}

struct CandScratch {
  std::vector<uint8_t> changed;
  std::vector<QEntry> added, lpt;
  std::vector<Seg> segs;
  std::vector<int> splits;
  SimScratch sim;
};

}  // namespace

Evaluation plan_search(const Problem& pb, const ModelParams& prm, const std::vector<int>& ref,
                       Evaluation* nosplit_out, const Evaluation* ref_ev) {
  const int B = (int)pb.seq_lens.size();
  const std::vector<int> lim = split_limits(pb, prm, ref);
  const Evaluation nosplit = simulate(pb, prm, std::vector<int>(B, 1));
  Evaluation cur = nosplit;
  SimPool& pool = sim_pool();

  std::vector<ReqRuns> runs(B);
  for (int b = 0; b < B; ++b) fill_runs(pb, prm, b, 1, runs[b]);
  bool decode_only = true;
  for (int b = 0; b < B; ++b) decode_only &= is_decode(pb.q_lens[b]);
  // Every candidate has a split, so candidates are queued longest first in
  // decode-only batches and chunk requests first otherwise. `base` is the
  // current plan's queue in that order (merged runs for longest first).
  std::vector<QEntry> base;
  if (decode_only) {
    for (int b = 0; b < B; ++b) base.insert(base.end(), runs[b].sorted[0].begin(), runs[b].sorted[0].end());
    std::stable_sort(base.begin(), base.end(), lpt_before);
  }
  auto fifo_segs = [&](const std::vector<uint8_t>* changed, std::vector<Seg>& segs) {
    segs.clear();
    auto seg = [&](int b) {
      const std::vector<QEntry>& v = runs[b].fifo[changed && (*changed)[b] ? 1 : 0];
      segs.push_back({v.data(), v.size()});
    };
    for (int b = 0; b < B; ++b)
      if (!is_decode(pb.q_lens[b])) seg(b);
    for (int b = 0; b < B; ++b)
      if (is_decode(pb.q_lens[b])) seg(b);
  };

  // Resume points: a candidate's queue agrees with `base` up to the first run
  // of a changed request (longest first: that request's first run in `base`,
  // before which no new run sorts; chunk first: the start of its segment), so
  // its run repeats the current plan's up to the first step that reads there.
  // The overlapped model keeps slot-release state outside the snapshot and
  // always runs in full.
  const bool resume = !prm.overlap_reduction;
  const int red_run = reduction_run(pb, prm);
  std::vector<int64_t> first_run(B, 0);
  Recording rec;
  SimScratch rec_sc;
  std::vector<Seg> base_segs;
  auto record = [&](std::vector<int>* tail) {
    if (decode_only) {
      std::fill(first_run.begin(), first_run.end(), -1);
      for (size_t i = 0; i < base.size(); ++i)
        if (first_run[base[i].req] < 0) first_run[base[i].req] = (int64_t)i;
      base_segs.assign(1, {base.data(), base.size()});
    } else {
      fifo_segs(nullptr, base_segs);
      int64_t pos = 0;
      for (const Seg& sg : base_segs) {
        first_run[sg.p[0].req] = pos;
        pos += (int64_t)sg.n;
      }
    }
    rec.thresholds.clear();
    for (int b = 0; b < B; ++b)
      if (cur.splits[b] < lim[b]) rec.thresholds.push_back(first_run[b]);
    std::sort(rec.thresholds.begin(), rec.thresholds.end());
    rec.thresholds.erase(std::unique(rec.thresholds.begin(), rec.thresholds.end()), rec.thresholds.end());
    return simulate_queue(pb, prm, cur.splits, base_segs.data(), base_segs.size(), rec_sc, tail,
                          nullptr, nullptr, resume ? &rec : nullptr, red_run);
  };
  if (resume) record(nullptr);

  // queue of cur with the requests in clist raised by one split; returns the
  // first run index at which it can differ from `base`
  auto build_cand = [&](const std::vector<int>& clist, CandScratch& cs) {
    cs.changed.assign(B, 0);
    cs.splits = cur.splits;
    int64_t p = INT64_MAX;
    for (int b : clist) {
      cs.changed[b] = 1;
      cs.splits[b] += 1;
      p = std::min(p, first_run[b]);
    }
    if (decode_only) {
      merge_lpt(base, runs, clist, cs.changed, cs.added, cs.lpt);
      cs.segs.assign(1, {cs.lpt.data(), cs.lpt.size()});
    } else {
      fifo_segs(&cs.changed, cs.segs);
    }
    return p;
  };
  // A chunk request's candidate (chunk-first order) changes the queue's first
  // segments, so the current plan's recording cannot shorten its run. It keeps
  // a recording of its own last full run instead, with snapshots before the
  // first run of every later segment: while the request's own count stays,
  // a later run agrees with the recorded queue up to the first segment whose
  // request has changed since, and resumes there (or repeats the recorded
  // result when none has). Each candidate touches only its own entry.
  struct OwnRecording {
    bool valid = false;
    std::vector<int> splits;   // the candidate's split counts when recorded
    Recording rec;
    SimResult res;
  };
  std::vector<OwnRecording> own(resume && !decode_only ? B : 0);
  auto eval_own = [&](int c, CandScratch& cs, const std::atomic<double>* cutoff) {
    OwnRecording& o = own[c];
    if (o.valid && o.splits[c] == cs.splits[c]) {
      int64_t pos = 0, p = -1;
      for (const Seg& sg : cs.segs) {
        const int r = sg.p[0].req;
        if (r != c && o.splits[r] != cs.splits[r]) {
          p = pos;
          break;
        }
        pos += (int64_t)sg.n;
      }
      if (p < 0) return o.res;
      const size_t k = std::lower_bound(o.rec.thresholds.begin(), o.rec.thresholds.end(), p) -
                       o.rec.thresholds.begin();
      if (k < o.rec.thresholds.size() && o.rec.thresholds[k] == p)
        return simulate_queue(pb, prm, cs.splits, cs.segs.data(), cs.segs.size(), cs.sim, nullptr,
                              &o.rec.snaps[o.rec.snap_of[k]], &o.rec, nullptr, red_run, cutoff);
    }
    // record a full run: thresholds at the segments after c's own
    o.rec.thresholds.clear();
    int64_t pos = 0;
    bool after = false;
    for (const Seg& sg : cs.segs) {
      if (after) o.rec.thresholds.push_back(pos);
      after |= sg.p[0].req == c;
      pos += (int64_t)sg.n;
    }
    o.res = simulate_queue(pb, prm, cs.splits, cs.segs.data(), cs.segs.size(), cs.sim, nullptr, nullptr,
                           nullptr, &o.rec, red_run);
    o.splits = cs.splits;
    o.valid = true;
    return o.res;
  };
  // cutoff (non-overlapped model): the best score found so far among this
  // round's candidates; a run that cannot beat it is cut (and not picked)
  auto eval_cand = [&](const std::vector<int>& clist, CandScratch& cs, bool use_snapshot,
                       const std::atomic<double>* cutoff) {
    const int64_t p = build_cand(clist, cs);
    if (use_snapshot && !own.empty() && clist.size() == 1 && !is_decode(pb.q_lens[clist[0]]))
      return eval_own(clist[0], cs, cutoff);
    const Snapshot* from = nullptr;
    if (use_snapshot) {
      const size_t k = std::lower_bound(rec.thresholds.begin(), rec.thresholds.end(), p) -
                       rec.thresholds.begin();
      from = &rec.snaps[rec.snap_of[k]];
    }
    return simulate_queue(pb, prm, cs.splits, cs.segs.data(), cs.segs.size(), cs.sim, nullptr, from,
                          from ? &rec : nullptr, nullptr, red_run, cutoff);
  };
  CandScratch adopt;

  // Lower bound on a candidate's score in the non-overlapped model.
  // Attention: a task of cost c takes at least rho c (tau >= rho), so it ends
  // no earlier than rho times the largest task cost (a request's first split,
  // which its last query token sees whole: ceil(tiles / s) + delta_attn); and
  // attention advances by at most K tile units per time unit (k / tau(k) <= K),
  // so it ends no earlier than the summed task cost over K. Reduction: every
  // unit starts after attention (the warps are released at its end), so the
  // score adds at least the largest unit cost and the summed unit cost over
  // K x W warps. A query tile's splits cover its visible tiles once, so a
  // request's task cost sums to KV heads x (visible tiles + delta_attn x
  // query tiles x splits).
  const bool bound = !prm.overlap_reduction;
  const std::vector<int64_t> vis_of = visible_tiles(pb, prm);
  std::vector<int64_t> tiles_of(B), qtiles_of(B);
  for (int b = 0; b < B; ++b) {
    tiles_of[b] = n_tiles(pb.seq_lens[b], prm.tile_tokens);
    qtiles_of[b] = num_qtiles(pb.q_lens[b], pb.query_tile);
  }
  auto task_max = [&](int b, int s) { return (double)((tiles_of[b] + s - 1) / s) + prm.delta_attn; };
  auto red_max = [&](int b, int s) {
    const int64_t rows = pb.q_lens[b] * (int64_t)pb.rows_per_token;
    const int64_t unit = rows >= red_run ? red_run : rows;
    return prm.delta_red + prm.gamma * (double)unit * (double)(s + pb.n_ext);
  };
  auto work_of = [&](int b, int s) {
    return (double)pb.num_kv_heads *
           ((double)vis_of[b] + prm.delta_attn * (double)qtiles_of[b] * (double)s);
  };
  auto red_of = [&](int b, int s) {
    const int64_t rows = pb.q_lens[b] * (int64_t)pb.rows_per_token;
    const double s_u = (double)(s + pb.n_ext);
    const int64_t full = rows / red_run, rem = rows % red_run;
    double r = (double)full * (prm.delta_red + prm.gamma * (double)red_run * s_u);
    if (rem > 0) r += prm.delta_red + prm.gamma * (double)rem * s_u;
    return r;
  };
  // the current plan's terms: totals, and the two largest per-request maxima
  // (a one-request candidate's maximum over the other requests is the
  // largest one not its own)
  struct Top2 {
    double v1 = -INFINITY, v2 = -INFINITY;
    int i1 = -1;
    void add(double v, int i) {
      if (v > v1) {
        v2 = v1;
        v1 = v;
        i1 = i;
      } else if (v > v2) {
        v2 = v;
      }
    }
    double without(int i) const { return i == i1 ? v2 : v1; }
  };
  Top2 t_top, r_top;
  double w_tot = 0, r_tot = 0;
  auto bound_terms = [&] {
    t_top = Top2{};
    r_top = Top2{};
    w_tot = r_tot = 0;
    for (int b = 0; b < B; ++b) {
      t_top.add(task_max(b, cur.splits[b]), b);
      r_top.add(red_max(b, cur.splits[b]), b);
      w_tot += work_of(b, cur.splits[b]);
      r_tot += red_of(b, cur.splits[b]);
    }
  };
  std::vector<uint8_t> in_cand(B, 0);
  auto cand_bound = [&](const std::vector<int>& clist) {
    double tm, rm, w = w_tot, r = r_tot;
    if (clist.size() == 1) {
      const int c = clist[0], s = cur.splits[c];
      tm = std::max(t_top.without(c), task_max(c, s + 1));
      rm = std::max(r_top.without(c), red_max(c, s + 1));
      w += work_of(c, s + 1) - work_of(c, s);
      r += red_of(c, s + 1) - red_of(c, s);
    } else {
      for (int b : clist) in_cand[b] = 1;
      tm = rm = -INFINITY;
      for (int b = 0; b < B; ++b) {
        const int s = cur.splits[b] + in_cand[b];
        tm = std::max(tm, task_max(b, s));
        rm = std::max(rm, red_max(b, s));
      }
      for (int b : clist) {
        w += work_of(b, cur.splits[b] + 1) - work_of(b, cur.splits[b]);
        r += red_of(b, cur.splits[b] + 1) - red_of(b, cur.splits[b]);
        in_cand[b] = 0;
      }
    }
    const double K = (double)prm.slots;
    return std::max(prm.rho * tm, w / K) + std::max(rm, r / (K * (double)prm.warps_per_slot));
  };

  for (;;) {
    // candidates in the pages' order: one more split for each request below
    // its limit, then the joint increment of the tied tail requests
    std::vector<std::vector<int>> cands;
    for (int b = 0; b < B; ++b)
      if (cur.splits[b] < lim[b]) cands.push_back({b});
    std::vector<int> tied;
    for (int b : cur.tail)
      if (cur.splits[b] < lim[b]) tied.push_back(b);
    if (tied.size() >= 2) cands.push_back(tied);
    if (cands.empty()) break;
    // Candidates are independent simulations: evaluate them on worker threads,
    // then pick in candidate order exactly as a sequential loop would. In the
    // non-overlapped model they are claimed in order of a lower bound on
    // their score, and one whose bound exceeds the best score found so far is
    // not simulated: it cannot be the pick (the key starts with the score).
    const size_t nc = cands.size();
    std::vector<SimResult> res(nc);
    std::vector<char> done(nc, 1);
    if (bound) {
      std::vector<double> lb(nc);
      std::vector<uint32_t> order(nc);
      bound_terms();
      for (size_t i = 0; i < nc; ++i) {
        lb[i] = cand_bound(cands[i]);
        order[i] = (uint32_t)i;
      }
      std::stable_sort(order.begin(), order.end(), [&](uint32_t x, uint32_t y) { return lb[x] < lb[y]; });
      std::fill(done.begin(), done.end(), 0);
      std::atomic<double> best_score{INFINITY};
      pool.run(nc, [&](size_t j) {
        const uint32_t i = order[j];
        const double bs = best_score.load();
        if (lb[i] > bs + 1e-9 * std::fabs(bs)) return;
        thread_local CandScratch cs;
        res[i] = eval_cand(cands[i], cs, resume, &best_score);
        if (res[i].cut) return;
        done[i] = 1;
        double c = best_score.load();
        while (res[i].score < c && !best_score.compare_exchange_weak(c, res[i].score)) {
        }
      });
    } else {
      pool.run(nc, [&](size_t i) {
        thread_local CandScratch cs;
        res[i] = eval_cand(cands[i], cs, resume, nullptr);
      });
    }
    const int64_t tot = cur.total_splits;
    auto key = [&](size_t i) {
      return std::make_tuple(res[i].score, res[i].t_attn, res[i].n_tasks,
                             tot + (int64_t)cands[i].size());
    };
    size_t best = nc;
    for (size_t i = 0; i < nc; ++i)
      if (done[i] && (best == nc || key(i) < key(best))) best = i;
    if (!(res[best].score < cur.score)) break;
    // adopt the best candidate: its runs and queue, then record its run (which
    // also gives its tail) for the next round's candidates
    build_cand(cands[best], adopt);
    if (decode_only) base.swap(adopt.lpt);
    std::vector<int> tail;
    cur.splits = adopt.splits;
    for (int b : cands[best]) {
      std::swap(runs[b].fifo[0], runs[b].fifo[1]);
      std::swap(runs[b].sorted[0], runs[b].sorted[1]);
      runs[b].s += 1;
      if (runs[b].s < lim[b]) {
        request_fifo(pb, prm, b, runs[b].s + 1, runs[b].fifo[1]);
        request_sorted(runs[b].fifo[1], runs[b].sorted[1]);
      }
    }
    const SimResult r = record(&tail);
    cur = to_eval(cur.splits, r, std::move(tail));
  }
  // final candidates in order: the search result, the reference plan, then
  // the proportional plans fitting 1..4 waves (when enabled); first best wins
  std::vector<std::vector<int>> finals;
  finals.push_back(ref);
  if (prm.balanced_candidates)
    for (int m = 1; m <= 4; ++m) {
      std::vector<int> c = balanced_plan(pb, prm, (int64_t)m * prm.slots);
      if (!c.empty()) finals.push_back(std::move(c));
    }
  Evaluation chosen = nosplit;
  bool chose_nosplit = true;
  if (key_less(cur, chosen)) {
    chosen = cur;
    chose_nosplit = false;
  }
  // a final candidate can only replace `chosen` with a score no larger than
  // its score: in the non-overlapped model a run that cannot is cut (and
  // skipped); the reference plan's evaluation is reused when given
  std::vector<Evaluation> fevs(finals.size());
  std::vector<char> fdone(finals.size(), 1);
  const std::atomic<double> fcut{chosen.score};
  pool.run(finals.size(), [&](size_t i) {
    if (i == 0 && ref_ev) {
      fevs[0] = *ref_ev;
    } else if (bound) {
      fdone[i] = simulate_below(pb, prm, finals[i], fcut, fevs[i]);
    } else {
      fevs[i] = simulate(pb, prm, finals[i]);
    }
  });
  for (size_t i = 0; i < fevs.size(); ++i) {
    Evaluation& ev = fevs[i];
    if (fdone[i] && key_less(ev, chosen)) {
      chosen = std::move(ev);
      chose_nosplit = false;
    }
  }
  if (!chose_nosplit && !(chosen.score <= (1.0 - prm.min_gain) * nosplit.score)) chosen = nosplit;
  if (nosplit_out) *nosplit_out = nosplit;
  return chosen;
}

}  // namespace skv
