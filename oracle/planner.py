"""Reference critical-wave split planner, a slow direct event simulation.

Test infrastructure only (see the package docstring). The library's C++ planner
must produce the same integers (split counts, ranges, task order) and the same
double-precision scores, bit for bit; this file is written independently from
the pages, in their order and notation.

What the pages fix (LiquidCP, section 5.2 "Critical-wave KV splitting"):

* Time unit: per-CTA time of one history KV tile with all K compute CTAs busy.
  With k attention CTAs active the per-tile time is tau(k) = max(rho, k / K)
  (Equation 5); every running attention task advances at rate 1 / tau(k), and k
  is updated whenever an attention task starts or finishes.
* An attention task t carries c_attn(t) = n_t + delta_attn tile-equivalents
  (n_t KV tiles plus a fixed per-task overhead).
* A history reduction u costs c_red(u) = delta_red + gamma * v_u * s_u
  (Equation 6): v_u output vectors (query token-head pairs), s_u contributing
  splits per vector.
* Attention tasks are dispatched in queue order to the first available CTA. A
  CTA releases its warps to reduction after its last attention task. Each
  reduction uses one warp and starts in queue order when its warp and its
  inputs are available. The score is the latest completion over attention and
  reduction; lower is better.
* Plan selection: start from NoSplit; each iteration evaluates +1 split on every
  sequence below its limit, plus a joint +1 for sequences whose tasks tie at the
  attention tail; accept the best candidate only if it improves the score; stop
  otherwise. Return the best of NoSplit, the search result and the reference
  plan; adopt a split plan only if it is at least 10% below NoSplit.
* Task ordering: split decode-only plans use longest-processing-time-first by
  c_attn; unsplit and mixed plans keep FIFO order, chunk tasks before history
  tasks ("Task ordering"; section 5.1 "Execution model").
* Appendix A.2 "Split planning": decode requests (at most 16 query tokens) with
  at least K local history tiles get a split limit of at least four; score ties
  favour earlier attention completion, then fewer attention tasks, then fewer
  total splits; reduction runs of output vectors are the largest run in
  {1, h_q, 2h_q, 4h_q, min(8h_q, 32)} that leaves at least 0.8 x (warps) tasks.

Readings where the pages are silent:

* Reference plan: the pages use FA3's native heuristic, which they do not give.
  FA3 splits every sequence of a batch the same number of times (Figure 8's
  FA3-derived plan (3, 3, 1) is one count, capped by the 2-tile request). The
  stand-in is that form: one batch-wide count u, request b gets min(u, n_b,
  max_splits) splits, and u in 1..max_splits is the one with the best model
  score (ties: the pages' keys, then the smaller u). Callers may inject an
  explicit reference plan instead.
* A split of n tiles into s parts gives the first (n mod s) parts ceil(n/s)
  tiles and the rest floor(n/s) (Figure 8 splits 176 tiles as 59, 59, 58).
* One attention task per (request, KV head, query tile, split); the pages fix
  one query tile per decoding region and size the tile by the rows it holds.
  A query tile is `query_tile` consecutive query tokens of a request (the last
  tile may hold fewer); the executor chooses the size (one token when each
  token's rows already fill a tile). A task's KV tiles are those its tile's
  last query token sees (causal rows: the most of any token of the tile).
* Events at equal times: completions first (in CTA order), then dispatches to
  the free CTAs in CTA-index order. Warps are claimed earliest-available first,
  ties by CTA then warp index. Candidate ties after the pages' keys: the earlier
  candidate (single increments in request order, then the joint increment).
* overlap_reduction = 0 (a separate merge launch): every warp becomes free at
  the last attention completion. overlap_reduction = 1: each CTA's warps become
  free when it finishes its last attention task (the fused engine of the pages).

Addition to the pages' candidate set (balanced_candidates = 1, the library's
default; 0 gives the pages' set exactly): the final choice also weighs four
proportional "balanced" plans, for m = 1..4 the plan with the smallest
per-split tile budget t whose attention tasks fit m waves of K slots (request
b gets min(ceil(n_b / t), n_b, max_splits) splits). The greedy +1 search cannot
reach such a plan when several requests' tasks must all shrink together; the
pages' reference plan plays this role for them, and the uniform stand-in above
does not. The candidates are scored by the same model and keys, so they change
the choice only when the model ranks one of them best.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field


@dataclass
class Params:
    tile_tokens: int = 64
    slots: int = 256            # K: concurrent attention workers
    warps_per_slot: int = 4     # warps each worker hands to reduction
    rho: float = 0.43
    delta_attn: float = 32.0
    delta_red: float = 2.5
    gamma: float = 0.47
    max_splits: int = 64
    min_gain: float = 0.10
    overlap_reduction: int = 0
    balanced_candidates: int = 1


@dataclass
class Problem:
    seq_lens: list
    q_lens: list
    num_kv_heads: int = 1       # attention tasks per query token and split
    rows_per_token: int = 1     # output vectors per query token (query heads)
    n_ext: int = 0              # external states merged into every row
    causal: bool = True
    query_tile: int = 1         # query tokens per attention task


@dataclass
class Task:
    b: int
    g: int
    qi: int       # query tile index within the request
    r: int
    lo: int       # first token of the split
    hi: int       # end token of the split (exclusive)
    n_t: int      # KV tiles of the split visible to this query token
    c: float      # c_attn


@dataclass
class Evaluation:
    splits: tuple
    score: float
    t_attn: float
    n_tasks: int
    total_splits: int
    tail: list = field(default_factory=list)   # requests whose attention ends at t_attn

    def key(self):
        return (self.score, self.t_attn, self.n_tasks, self.total_splits)


def n_tiles(L: int, T: int) -> int:
    return (L + T - 1) // T


def split_tiles(n: int, s: int):
    """Tile ranges of n tiles in s parts: the first n mod s parts are one tile longer."""
    q, rem = divmod(n, s)
    out, start = [], 0
    for r in range(s):
        size = q + (1 if r < rem else 0)
        out.append((start, start + size))
        start += size
    return out


def split_ranges(L: int, s: int, T: int):
    """Token ranges [lo, hi) of the s splits of a history of L tokens."""
    return [(a * T, min(e * T, L)) for a, e in split_tiles(n_tiles(L, T), s)]


def is_decode(n: int) -> bool:
    return n <= 16


def query_tiles(n: int, qt: int):
    """(first, last) query token of each tile of a request with n tokens."""
    return [(a, min(n, a + qt) - 1) for a in range(0, n, qt)]


def build_tasks(pb: Problem, prm: Params, splits):
    """Attention tasks of a plan in queue order."""
    T = prm.tile_tokens
    B = len(pb.seq_lens)
    fifo = []
    for b in range(B):
        L, n = pb.seq_lens[b], pb.q_lens[b]
        rng = split_ranges(L, splits[b], T)
        for qi, (_, last) in enumerate(query_tiles(n, pb.query_tile)):
            vis = L - n + last + 1 if pb.causal else L
            vis_t = n_tiles(vis, T)
            for g in range(pb.num_kv_heads):
                for r, (lo, hi) in enumerate(rng):
                    lo_t, hi_t = lo // T, n_tiles(hi, T)
                    n_t = max(0, min(hi_t, vis_t) - lo_t)
                    fifo.append(Task(b, g, qi, r, lo, hi, n_t, n_t + prm.delta_attn))
    decode_only = all(is_decode(n) for n in pb.q_lens)
    if decode_only and any(s > 1 for s in splits):
        # stable: equal costs keep FIFO order
        return sorted(fifo, key=lambda t: -t.c)
    if not decode_only:
        chunk = [t for t in fifo if not is_decode(pb.q_lens[t.b])]
        hist = [t for t in fifo if is_decode(pb.q_lens[t.b])]
        return chunk + hist
    return fifo


def reduction_run(pb: Problem, prm: Params) -> int:
    """Rows per reduction unit: the largest run in {1, h, 2h, 4h, min(8h, 32)}
    that leaves at least 0.8 x (K x warps) units (h = rows per query token)."""
    h = pb.rows_per_token
    warps = prm.slots * prm.warps_per_slot
    best = 1
    for run in (1, h, 2 * h, 4 * h, min(8 * h, 32)):
        units = sum((n * h + run - 1) // run for n in pb.q_lens)
        if units >= 0.8 * warps and run > best:
            best = run
    return best


def reduction_units(pb: Problem, prm: Params, splits):
    """(request, c_red) of every reduction unit in queue order."""
    run = reduction_run(pb, prm)
    units = []
    for b, n in enumerate(pb.q_lens):
        rows = n * pb.rows_per_token
        s_u = splits[b] + pb.n_ext
        start = 0
        while start < rows:
            v = min(run, rows - start)
            units.append((b, prm.delta_red + prm.gamma * v * s_u))
            start += v
    return units


def simulate(pb: Problem, prm: Params, splits) -> Evaluation:
    """Critical-wave simulation of one plan."""
    tasks = build_tasks(pb, prm, splits)
    K = prm.slots
    B = len(pb.seq_lens)
    t = 0.0          # model time
    vw = 0.0         # work done so far by any running task (integral of 1/tau)
    running = []     # heap of (finish work, slot, task index)
    free = list(range(K))
    heapq.heapify(free)
    done = [0.0] * B
    release = [0.0] * K
    nxt = 0
    while free and nxt < len(tasks):
        s = heapq.heappop(free)
        heapq.heappush(running, (vw + tasks[nxt].c, s, nxt))
        nxt += 1
    while running:
        tau = max(prm.rho, len(running) / K)
        fw = running[0][0]
        t = t + (fw - vw) * tau
        vw = fw
        freed = []
        while running and running[0][0] == fw:
            _, s, i = heapq.heappop(running)
            b = tasks[i].b
            if t > done[b]:
                done[b] = t
            freed.append(s)
        for s in freed:
            heapq.heappush(free, s)
        while free and nxt < len(tasks):
            s = heapq.heappop(free)
            heapq.heappush(running, (vw + tasks[nxt].c, s, nxt))
            nxt += 1
        for s in freed:
            release[s] = t          # overwritten if the slot is dispatched again later
    t_attn = t
    # a slot dispatched again is not idle: its release is its later completion,
    # which the loop above records when that task finishes.
    if prm.overlap_reduction:
        warps = [(release[s], s, w) for s in range(K) for w in range(prm.warps_per_slot)]
    else:
        warps = [(t_attn, s, w) for s in range(K) for w in range(prm.warps_per_slot)]
    heapq.heapify(warps)
    score = t_attn
    for b, c in reduction_units(pb, prm, splits):
        avail, s, w = heapq.heappop(warps)
        start = avail if avail > done[b] else done[b]
        end = start + c
        heapq.heappush(warps, (end, s, w))
        if end > score:
            score = end
    tail = [b for b in range(B) if done[b] == t_attn]
    return Evaluation(tuple(splits), score, t_attn, len(tasks), sum(splits), tail)


def uniform_plan(pb: Problem, prm: Params, u: int):
    """One batch-wide split count u, capped per request by its tiles and max_splits."""
    T = prm.tile_tokens
    return [max(1, min(u, n_tiles(L, T), prm.max_splits)) for L in pb.seq_lens]


def reference_plan(pb: Problem, prm: Params):
    """Stand-in for the pages' FA3-derived reference plan: the batch-wide count
    with the best model score."""
    best, best_u = None, 1
    for u in range(1, prm.max_splits + 1):
        ev = simulate(pb, prm, uniform_plan(pb, prm, u))
        if best is None or ev.key() < best.key():
            best, best_u = ev, u
    return uniform_plan(pb, prm, best_u)


def balanced_plan(pb: Problem, prm: Params, wave_tasks: int):
    """Proportional plan: the smallest per-split tile budget t whose plan has at
    most wave_tasks attention tasks, request b getting min(ceil(n_b / t), n_b,
    max_splits) splits (at least one); None if even NoSplit has more tasks."""
    T = prm.tile_tokens
    nt = [n_tiles(L, T) for L in pb.seq_lens]
    # tasks of one split: one per query tile and KV head
    per_split = [len(query_tiles(n, pb.query_tile)) * pb.num_kv_heads for n in pb.q_lens]

    def counts(t):
        return [max(1, min(-(-n // t), n, prm.max_splits)) for n in nt]

    def tasks(c):
        return sum(s * m for s, m in zip(c, per_split))

    hi = max(max(nt), 1)
    if tasks(counts(hi)) > wave_tasks:
        return None
    lo = 1
    while lo < hi:   # tasks(counts(t)) does not increase with t
        mid = (lo + hi) // 2
        if tasks(counts(mid)) <= wave_tasks:
            hi = mid
        else:
            lo = mid + 1
    return counts(lo)


def split_limits(pb: Problem, prm: Params, ref):
    """Per-request search limits: the reference counts, raised to at least four
    for decode requests with at least K tiles, capped by tiles and max_splits."""
    T = prm.tile_tokens
    out = []
    for b, L in enumerate(pb.seq_lens):
        nt = n_tiles(L, T)
        u = ref[b]
        if is_decode(pb.q_lens[b]) and nt >= prm.slots:
            u = max(u, 4)
        out.append(max(1, min(u, nt, prm.max_splits)))
    return out


def plan(pb: Problem, prm: Params, ref=None, trace=None):
    """Greedy critical-wave search; returns the chosen Evaluation.

    ``trace`` (a list) receives the accepted evaluations in search order.
    """
    B = len(pb.seq_lens)
    ref = list(reference_plan(pb, prm) if ref is None else ref)
    lim = split_limits(pb, prm, ref)
    nosplit = simulate(pb, prm, [1] * B)
    cur = nosplit
    if trace is not None:
        trace.append(cur)
    while True:
        cands = []
        for b in range(B):
            if cur.splits[b] < lim[b]:
                s = list(cur.splits)
                s[b] += 1
                cands.append(s)
        tied = [b for b in cur.tail if cur.splits[b] < lim[b]]
        if len(tied) >= 2:
            s = list(cur.splits)
            for b in tied:
                s[b] += 1
            cands.append(s)
        if not cands:
            break
        best = None
        for s in cands:
            ev = simulate(pb, prm, s)
            if best is None or ev.key() < best.key():
                best = ev
        if best.score < cur.score:
            cur = best
            if trace is not None:
                trace.append(cur)
        else:
            break
    cands = [cur, simulate(pb, prm, ref)]
    if prm.balanced_candidates:
        for m in (1, 2, 3, 4):
            c = balanced_plan(pb, prm, m * prm.slots)
            if c is not None:
                cands.append(simulate(pb, prm, c))
    chosen = nosplit
    for ev in cands:
        if ev.key() < chosen.key():
            chosen = ev
    if chosen is not nosplit and not chosen.score <= (1.0 - prm.min_gain) * nosplit.score:
        chosen = nosplit
    return chosen
