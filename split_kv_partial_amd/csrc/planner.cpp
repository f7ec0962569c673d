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
#include <cmath>
#include <cstdint>
#include <numeric>
#include <queue>
#include <thread>
#include <tuple>
#include <vector>

#include "internal.hpp"

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

// Tasks of a plan in queue order: FIFO enumerates (request, query token, KV head,
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
  for (int b = 0; b < B; ++b) {
    const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
    for (int64_t qi = 0; qi < n; ++qi) {
      const int64_t vis = pb.causal ? L - n + qi + 1 : L;
      const int64_t vis_t = n_tiles(vis, T);
      for (int g = 0; g < pb.num_kv_heads; ++g) {
        for (int r = 0; r < (int)ranges[b].size(); ++r) {
          const int64_t lo = ranges[b][r].first, hi = ranges[b][r].second;
          const int64_t lo_t = lo / T, hi_t = n_tiles(hi, T);
          const int64_t nt = std::max<int64_t>(0, std::min(hi_t, vis_t) - lo_t);
          TaskDesc t{b, g, (int32_t)qi, r, (int32_t)lo, (int32_t)hi,
                     (int32_t)(qoff[b] + qi), 0};
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

// Min-heap entries ordered exactly like the reference's tuples.
struct Running {
  double fw;
  int slot;
  int64_t idx;
  bool operator>(const Running& o) const {
    return std::tie(fw, slot, idx) > std::tie(o.fw, o.slot, o.idx);
  }
};
struct Warp {
  double avail;
  int slot, w;
  bool operator>(const Warp& o) const {
    return std::tie(avail, slot, w) > std::tie(o.avail, o.slot, o.w);
  }
};
template <class T>
using MinHeap = std::priority_queue<T, std::vector<T>, std::greater<T>>;

}  // namespace

Evaluation simulate(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits) {
  const int B = (int)pb.seq_lens.size();
  const int K = prm.slots;
  std::vector<std::vector<std::pair<int64_t, int64_t>>> ranges(B);
  for (int b = 0; b < B; ++b) ranges[b] = split_ranges(pb.seq_lens[b], splits[b], prm.tile_tokens);
  std::vector<TaskDesc> tasks;
  std::vector<double> cost;
  build_tasks(pb, prm, ranges, tasks, &cost);
  const int64_t nt = (int64_t)tasks.size();

  double t = 0.0, vw = 0.0;
  MinHeap<Running> running;
  MinHeap<int> free_slots;
  for (int s = 0; s < K; ++s) free_slots.push(s);
  std::vector<double> done(B, 0.0), release(K, 0.0);
  int64_t nxt = 0;
  while (!free_slots.empty() && nxt < nt) {
    int s = free_slots.top();
    free_slots.pop();
    running.push({vw + cost[nxt], s, nxt});
    ++nxt;
  }
  std::vector<int> freed;
  while (!running.empty()) {
    const double tau = std::max(prm.rho, (double)running.size() / (double)K);
    const double fw = running.top().fw;
    t = t + (fw - vw) * tau;
    vw = fw;
    freed.clear();
    while (!running.empty() && running.top().fw == fw) {
      Running r = running.top();
      running.pop();
      const int b = tasks[r.idx].b;
      if (t > done[b]) done[b] = t;
      freed.push_back(r.slot);
    }
    for (int s : freed) free_slots.push(s);
    while (!free_slots.empty() && nxt < nt) {
      int s = free_slots.top();
      free_slots.pop();
      running.push({vw + cost[nxt], s, nxt});
      ++nxt;
    }
    for (int s : freed) release[s] = t;
  }
  const double t_attn = t;

  // Reduction phase. Warps are claimed earliest-available first (ties by slot,
  // then warp). Without overlap every warp becomes free at t_attn, when every
  // request's inputs are ready, so the first K*W units start exactly at t_attn
  // on warps taken in (slot, warp) order; only later units need the heap.
  const int run = reduction_run(pb, prm);
  const int64_t nwarps = (int64_t)K * prm.warps_per_slot;
  double score = t_attn;
  // The shortcut needs every claimed warp to end strictly after t_attn, so that
  // no used warp can tie with an untouched one: the cheapest unit costs at least
  // delta_red + gamma (v_u >= 1, s_u >= 1).
  const bool fast = !prm.overlap_reduction && t_attn + (prm.delta_red + prm.gamma) > t_attn;
  std::vector<Warp> wv;
  int64_t claimed = 0;
  MinHeap<Warp> warps;
  if (!fast) {
    wv.reserve((size_t)nwarps);
    for (int s = 0; s < K; ++s)
      for (int w = 0; w < prm.warps_per_slot; ++w)
        wv.push_back({prm.overlap_reduction ? release[s] : t_attn, s, w});
    warps = MinHeap<Warp>(std::greater<Warp>(), std::move(wv));
  }
  for (int b = 0; b < B; ++b) {
    const int64_t rows = pb.q_lens[b] * (int64_t)pb.rows_per_token;
    const int64_t s_u = splits[b] + pb.n_ext;
    for (int64_t start = 0; start < rows;) {
      const int64_t v = std::min<int64_t>(run, rows - start);
      const double c = prm.delta_red + prm.gamma * (double)v * (double)s_u;
      Warp w;
      if (fast && claimed < nwarps) {
        // still-untouched warp number `claimed`: available at t_attn
        w = {t_attn, (int)(claimed / prm.warps_per_slot), (int)(claimed % prm.warps_per_slot)};
        ++claimed;
      } else {
        w = warps.top();
        warps.pop();
      }
      const double st = w.avail > done[b] ? w.avail : done[b];
      const double end = st + c;
      warps.push({end, w.slot, w.w});
      if (end > score) score = end;
      start += v;
    }
  }
  Evaluation ev;
  ev.splits = splits;
  ev.score = score;
  ev.t_attn = t_attn;
  ev.n_tasks = nt;
  ev.total_splits = std::accumulate(splits.begin(), splits.end(), (int64_t)0);
  for (int b = 0; b < B; ++b)
    if (done[b] == t_attn) ev.tail.push_back(b);
  return ev;
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

// Stand-in for the pages' FA3-derived reference plan (FA3's heuristic is not
// given): one batch-wide split count, capped per request by its tiles, chosen
// by the model among 1..max_splits (ties: the pages' keys, then the smaller
// count). Counts are simulated on worker threads; the pick is sequential.
std::vector<int> reference_plan(const Problem& pb, const ModelParams& prm) {
  const int U = prm.max_splits;
  std::vector<Evaluation> evs(U);
  const unsigned nthreads = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  {
    std::vector<std::thread> pool;
    for (unsigned t = 0; t < nthreads; ++t)
      pool.emplace_back([&, t]() {
        for (int u = 1 + (int)t; u <= U; u += (int)nthreads) evs[u - 1] = simulate(pb, prm, uniform_plan(pb, prm, u));
      });
    for (auto& th : pool) th.join();
  }
  int best_u = 1;
  for (int u = 2; u <= U; ++u)
    if (key_less(evs[u - 1], evs[best_u - 1])) best_u = u;
  return uniform_plan(pb, prm, best_u);
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

Evaluation plan_search(const Problem& pb, const ModelParams& prm, const std::vector<int>& ref,
                       Evaluation* nosplit_out) {
  const int B = (int)pb.seq_lens.size();
  const std::vector<int> lim = split_limits(pb, prm, ref);
  const Evaluation nosplit = simulate(pb, prm, std::vector<int>(B, 1));
  Evaluation cur = nosplit;
  for (;;) {
    std::vector<std::vector<int>> cands;
    for (int b = 0; b < B; ++b) {
      if (cur.splits[b] < lim[b]) {
        std::vector<int> s = cur.splits;
        s[b] += 1;
        cands.push_back(std::move(s));
      }
    }
    std::vector<int> tied;
    for (int b : cur.tail)
      if (cur.splits[b] < lim[b]) tied.push_back(b);
    if (tied.size() >= 2) {
      std::vector<int> s = cur.splits;
      for (int b : tied) s[b] += 1;
      cands.push_back(std::move(s));
    }
    if (cands.empty()) break;
    // Candidates are independent simulations: evaluate them on worker threads,
    // then pick in candidate order exactly as a sequential loop would.
    std::vector<Evaluation> evs(cands.size());
    const size_t nthreads =
        std::min<size_t>(cands.size(), std::max(1u, std::min(16u, std::thread::hardware_concurrency())));
    if (nthreads <= 1 || cands.size() < 4) {
      for (size_t i = 0; i < cands.size(); ++i) evs[i] = simulate(pb, prm, cands[i]);
    } else {
      std::vector<std::thread> pool;
      for (size_t t = 0; t < nthreads; ++t)
        pool.emplace_back([&, t]() {
          for (size_t i = t; i < cands.size(); i += nthreads) evs[i] = simulate(pb, prm, cands[i]);
        });
      for (auto& th : pool) th.join();
    }
    bool have = false;
    Evaluation best;
    for (auto& ev : evs) {
      if (!have || key_less(ev, best)) {
        best = std::move(ev);
        have = true;
      }
    }
    if (best.score < cur.score)
      cur = std::move(best);
    else
      break;
  }
  Evaluation chosen = nosplit;
  bool chose_nosplit = true;
  for (int k = 0; k < 2; ++k) {
    Evaluation ev = k == 0 ? cur : simulate(pb, prm, ref);
    if (key_less(ev, chosen)) {
      chosen = std::move(ev);
      chose_nosplit = false;
    }
  }
  if (!chose_nosplit && !(chosen.score <= (1.0 - prm.min_gain) * nosplit.score)) chosen = nosplit;
  if (nosplit_out) *nosplit_out = nosplit;
  return chosen;
}

}  // namespace skv
