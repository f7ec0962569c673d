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
#include <condition_variable>
#include <functional>
#include <mutex>
#include <cmath>
#include <cstdint>
#include <map>
#include <numeric>
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

struct SimScratch {
  std::vector<double> cost;       // attention task costs in queue order
  std::vector<int32_t> req;       // request of each queued task
  std::vector<double> fifo_cost;
  std::vector<int32_t> fifo_req;
  std::vector<uint32_t> order;
  std::vector<double> done_fw, ev_fw, ev_t, done;
  std::vector<Group> heap;
};

// Queue of attention tasks (cost and request), in the order build_tasks gives.
static void queue_costs(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits,
                        SimScratch& sc) {
  const int T = prm.tile_tokens;
  const int B = (int)pb.seq_lens.size();
  bool any_split = false, decode_only = true;
  for (int b = 0; b < B; ++b) {
    any_split |= splits[b] > 1;
    decode_only &= is_decode(pb.q_lens[b]);
  }
  sc.fifo_cost.clear();
  sc.fifo_req.clear();
  for (int b = 0; b < B; ++b) {
    const int64_t L = pb.seq_lens[b], n = pb.q_lens[b];
    const int64_t total = n_tiles(L, T);
    const int s = splits[b];
    for (int64_t qi = 0; qi < n; ++qi) {
      const int64_t vis = pb.causal ? L - n + qi + 1 : L;
      const int64_t vis_t = n_tiles(vis, T);
      for (int g = 0; g < pb.num_kv_heads; ++g) {
        // the same tile split as split_ranges: the first total mod s parts
        // are one tile longer
        int64_t lo_t = 0;
        for (int r = 0; r < s; ++r) {
          const int64_t len = total / s + (r < total % s ? 1 : 0);
          const int64_t hi_t = lo_t + len;
          const int64_t nt = std::max<int64_t>(0, std::min(hi_t, vis_t) - lo_t);
          sc.fifo_cost.push_back((double)nt + prm.delta_attn);
          sc.fifo_req.push_back(b);
          lo_t = hi_t;
        }
      }
    }
  }
  const size_t N = sc.fifo_cost.size();
  sc.order.resize(N);
  std::iota(sc.order.begin(), sc.order.end(), 0u);
  if (decode_only && any_split) {
    const double* c = sc.fifo_cost.data();
    std::stable_sort(sc.order.begin(), sc.order.end(), [c](uint32_t x, uint32_t y) { return c[x] > c[y]; });
  } else if (!decode_only) {
    const int32_t* r = sc.fifo_req.data();
    std::stable_partition(sc.order.begin(), sc.order.end(),
                          [&](uint32_t x) { return !is_decode(pb.q_lens[r[x]]); });
  }
  sc.cost.resize(N);
  sc.req.resize(N);
  for (size_t i = 0; i < N; ++i) {
    sc.cost[i] = sc.fifo_cost[sc.order[i]];
    sc.req[i] = sc.fifo_req[sc.order[i]];
  }
}

}  // namespace

Evaluation simulate(const Problem& pb, const ModelParams& prm, const std::vector<int>& splits) {
  thread_local SimScratch sc;
  const int B = (int)pb.seq_lens.size();
  const int64_t K = prm.slots;
  queue_costs(pb, prm, splits, sc);
  const int64_t nt = (int64_t)sc.cost.size();
  const double* cost = sc.cost.data();
  const int32_t* req = sc.req.data();

  // ---- attention phase ----
  sc.done_fw.assign(B, 0.0);
  sc.ev_fw.clear();
  sc.ev_t.clear();
  sc.heap.clear();
  std::map<double, int64_t> release;  // slot release times (for overlapped reductions)
  auto heap_push = [&](double fw, int64_t n) {
    sc.heap.push_back({fw, n});
    std::push_heap(sc.heap.begin(), sc.heap.end(), std::greater<Group>());
  };
  double t = 0.0, vw = 0.0;
  int64_t running = 0, nxt = 0;
  // start up to `free_slots` queued tasks at work clock vw; returns how many started
  auto start_tasks = [&](int64_t free_slots) {
    int64_t started = 0;
    while (started < free_slots && nxt < nt) {
      const double c = cost[nxt];
      int64_t j = nxt + 1;
      const int64_t lim = nxt + (free_slots - started);
      while (j < lim && j < nt && cost[j] == c) ++j;
      const double fw = vw + c;
      for (int64_t i = nxt; i < j; ++i)
        if (fw > sc.done_fw[req[i]]) sc.done_fw[req[i]] = fw;
      heap_push(fw, j - nxt);
      started += j - nxt;
      nxt = j;
    }
    running += started;
    return started;
  };
  start_tasks(K);
  if (K > nt) release[0.0] += (K - nt) * prm.warps_per_slot;
  while (!sc.heap.empty()) {
    const double tau = std::max(prm.rho, (double)running / (double)K);
    const double fw = sc.heap.front().fw;
    t = t + (fw - vw) * tau;
    vw = fw;
    int64_t m = 0;
    while (!sc.heap.empty() && sc.heap.front().fw == fw) {
      m += sc.heap.front().n;
      std::pop_heap(sc.heap.begin(), sc.heap.end(), std::greater<Group>());
      sc.heap.pop_back();
    }
    running -= m;
    sc.ev_fw.push_back(fw);
    sc.ev_t.push_back(t);
    const int64_t started = start_tasks(m);
    if (m > started) release[t] += (m - started) * prm.warps_per_slot;
  }
  const double t_attn = t;
  // a request's attention ends at the event of its latest-finishing task
  sc.done.assign(B, 0.0);
  for (int b = 0; b < B; ++b) {
    const double f = sc.done_fw[b];
    if (f == 0.0) continue;  // no task started (cannot happen: every request has one)
    const auto it = std::lower_bound(sc.ev_fw.begin(), sc.ev_fw.end(), f);
    sc.done[b] = sc.ev_t[it - sc.ev_fw.begin()];
  }

  // ---- reduction phase: units in request order, each on the earliest-free warp ----
  const int run = reduction_run(pb, prm);
  const int64_t nwarps = K * prm.warps_per_slot;
  std::map<double, int64_t> warps;
  if (prm.overlap_reduction)
    warps = std::move(release);
  else
    warps[t_attn] = nwarps;
  double score = t_attn;
  auto assign = [&](int64_t k, double c, double d) {
    while (k > 0) {
      auto it = warps.begin();
      const double a = it->first;
      const int64_t avail = it->second;
      const double st = a > d ? a : d;
      const double end = st + c;
      const int64_t j = std::min(k, avail);
      if (j == avail)
        warps.erase(it);
      else
        it->second -= j;
      warps[end] += j;
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
  Evaluation ev;
  ev.splits = splits;
  ev.score = score;
  ev.t_attn = t_attn;
  ev.n_tasks = nt;
  ev.total_splits = std::accumulate(splits.begin(), splits.end(), (int64_t)0);
  for (int b = 0; b < B; ++b)
    if (sc.done[b] == t_attn) ev.tail.push_back(b);
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

// Worker threads for independent simulations. The caller takes part; each
// index is run exactly once and results are written by index, so the outcome
// does not depend on which thread ran what.
class SimPool {
 public:
  SimPool() {
    const unsigned hw = std::thread::hardware_concurrency();
    const unsigned n = std::max(1u, std::min(16u, hw));
    for (unsigned i = 1; i < n; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~SimPool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& w : workers_) w.join();
  }
  size_t threads() const { return workers_.size() + 1; }
  void run(size_t count, const std::function<void(size_t)>& fn) {
    if (count == 0) return;
    if (workers_.empty() || count < 4) {
      for (size_t i = 0; i < count; ++i) fn(i);
      return;
    }
    {
      std::lock_guard<std::mutex> g(mu_);
      fn_ = &fn;
      count_ = count;
      next_.store(0);
      pending_ = count;
      ++gen_;
    }
    cv_.notify_all();
    work();
    std::unique_lock<std::mutex> g(mu_);
    done_cv_.wait(g, [this] { return pending_ == 0; });
    fn_ = nullptr;
  }

 private:
  void work() {
    size_t finished = 0;
    for (;;) {
      const size_t i = next_.fetch_add(1);
      if (i >= count_) break;
      (*fn_)(i);
      ++finished;
    }
    if (finished) {
      std::lock_guard<std::mutex> g(mu_);
      pending_ -= finished;
      if (pending_ == 0) done_cv_.notify_all();
    }
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> g(mu_);
        cv_.wait(g, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
      }
      work();
    }
  }
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(size_t)>* fn_ = nullptr;
  size_t count_ = 0, pending_ = 0;
  std::atomic<size_t> next_{0};
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// Stand-in for the pages' FA3-derived reference plan (FA3's heuristic is not
// given): one batch-wide split count, capped per request by its tiles, chosen
// by the model among 1..max_splits (ties: the pages' keys, then the smaller
// count). Counts are simulated on worker threads; the pick is sequential.
std::vector<int> reference_plan(const Problem& pb, const ModelParams& prm) {
  const int U = prm.max_splits;
  std::vector<Evaluation> evs(U);
  SimPool pool;
  pool.run((size_t)U, [&](size_t i) { evs[i] = simulate(pb, prm, uniform_plan(pb, prm, (int)i + 1)); });
  int best_u = 1;
  for (int u = 2; u <= U; ++u)
    if (key_less(evs[u - 1], evs[best_u - 1])) best_u = u;
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
    per_split[b] = pb.q_lens[b] * (int64_t)pb.num_kv_heads;
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

Evaluation plan_search(const Problem& pb, const ModelParams& prm, const std::vector<int>& ref,
                       Evaluation* nosplit_out) {
  const int B = (int)pb.seq_lens.size();
  const std::vector<int> lim = split_limits(pb, prm, ref);
  const Evaluation nosplit = simulate(pb, prm, std::vector<int>(B, 1));
  Evaluation cur = nosplit;
  SimPool pool;
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
    pool.run(cands.size(), [&](size_t i) { evs[i] = simulate(pb, prm, cands[i]); });
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
  // final candidates in order: the search result, the reference plan, then
  // the proportional plans fitting 1..4 waves (when enabled); first best wins
  std::vector<std::vector<int>> finals;
  finals.push_back(ref);
  if (prm.balanced_candidates)
    for (int m = 1; m <= 4; ++m) {
      std::vector<int> c = balanced_plan(pb, prm, (int64_t)m * prm.slots);
      if (!c.empty()) finals.push_back(std::move(c));
    }
  std::vector<Evaluation> fevs(finals.size());
  pool.run(finals.size(), [&](size_t i) { fevs[i] = simulate(pb, prm, finals[i]); });
  Evaluation chosen = nosplit;
  bool chose_nosplit = true;
  if (key_less(cur, chosen)) {
    chosen = cur;
    chose_nosplit = false;
  }
  for (auto& ev : fevs) {
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
