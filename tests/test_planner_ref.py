"""Pins for the reference critical-wave planner (CPU only).

The exact pin is LiquidCP Figure 8 (section 5.2; fixture under tests/golden/):
histories of 192, 176 and 2 KV tiles on K = 4 CTAs with delta_attn = delta_red = 4,
gamma = 1, rho = 3/4 and v_u = 1 score 152 (NoSplit), 121.5 (FA3-derived (3,3,1))
and 104 (chosen (2,2,1)). The remaining tests check closed forms of the model
and invariants that every plan must satisfy.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import planner as PL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fig8_critical_wave.json")


def fig8():
    g = json.load(open(GOLDEN))
    T = 64
    pb = PL.Problem(seq_lens=[t * T for t in g["histories_tiles"]], q_lens=[1, 1, 1])
    p = g["parameters"]
    prm = PL.Params(tile_tokens=T, slots=p["K"], warps_per_slot=1, rho=p["rho"],
                    delta_attn=p["delta_attn"], delta_red=p["delta_red"], gamma=p["gamma"],
                    overlap_reduction=1)
    return g, pb, prm


def test_fig8_printed_scores():
    g, pb, prm = fig8()
    pr = g["printed"]
    assert PL.simulate(pb, prm, [1, 1, 1]).score == pr["NoSplit (1,1,1)"]
    assert PL.simulate(pb, prm, [3, 3, 1]).score == pr["FA3-derived (3,3,1)"]
    assert PL.simulate(pb, prm, [2, 2, 1]).score == pr["critical-wave (2,2,1)"]


def test_fig8_split_sizes():
    g, _, _ = fig8()
    sizes = g["printed_split_sizes"]
    assert [e - a for a, e in PL.split_tiles(176, 3)] == sizes["S1 176 tiles in 3 parts"]
    assert [e - a for a, e in PL.split_tiles(192, 2)] == sizes["S0 192 tiles in 2 parts"]
    assert [e - a for a, e in PL.split_tiles(176, 2)] == sizes["S1 176 tiles in 2 parts"]


def test_fig8_search_path_and_choice():
    # Hand derivation under the model (all four CTAs busy give tau = 1, fewer give
    # tau = 3/4):
    #  (2,1,1): tasks 180,100,100,6 -> the 6-task ends at 6, then three run at 3/4:
    #           100-tasks end at 6 + 94*0.75 = 76.5, the 180-task at 6 + 174*0.75 = 136.5;
    #           S1's reduction (4 + 1) ends at 141.5.
    #  (2,2,1): 100,100,92,92 at tau 1 until 92, then 6 and the two 100-tails at 3/4:
    #           S0 ready at 98, reduction 4 + 2 -> 104.
    #  (3,2,1): 127.5 and (2,3,1): 118 do not improve 104, so the search stops.
    g, pb, prm = fig8()
    tr = []
    ch = PL.plan(pb, prm, ref=g["reference_plan"], trace=tr)
    assert [(e.splits, e.score) for e in tr] == [((1, 1, 1), 152.0), ((2, 1, 1), 141.5),
                                                  ((2, 2, 1), 104.0)]
    assert PL.simulate(pb, prm, [3, 2, 1]).score == 127.5
    assert PL.simulate(pb, prm, [2, 3, 1]).score == 118.0
    assert list(ch.splits) == g["chosen"]
    assert PL.split_limits(pb, prm, g["reference_plan"]) == [4, 4, 1]


def test_fig8_score_independent_of_warps_per_cta():
    g, pb, prm = fig8()
    for W in (1, 2, 12):
        prm.warps_per_slot = W
        assert PL.simulate(pb, prm, [2, 2, 1]).score == 104.0
        assert PL.simulate(pb, prm, [3, 3, 1]).score == 121.5


def test_single_task_closed_form():
    # one task alone: tau = max(rho, 1/K); score = (n + delta_attn) tau + delta_red + gamma v s
    for K, rho in [(4, 0.43), (1, 0.43), (8, 0.9)]:
        prm = PL.Params(slots=K, warps_per_slot=1, rho=rho, delta_attn=32, delta_red=2.5,
                        gamma=0.47)
        pb = PL.Problem(seq_lens=[640], q_lens=[1], rows_per_token=1)
        ev = PL.simulate(pb, prm, [1])
        tau = max(rho, 1 / K)
        assert math.isclose(ev.t_attn, 42 * tau, rel_tol=0, abs_tol=1e-12)
        assert math.isclose(ev.score, 42 * tau + 2.5 + 0.47, rel_tol=0, abs_tol=1e-12)


def test_full_wave_equal_tasks():
    # K equal tasks on K CTAs: k = K throughout, tau = 1, t_attn = c
    K = 16
    prm = PL.Params(slots=K, warps_per_slot=2, rho=0.5, delta_attn=8)
    pb = PL.Problem(seq_lens=[64 * 10] * 4, q_lens=[1] * 4, num_kv_heads=4, rows_per_token=4)
    ev = PL.simulate(pb, prm, [1, 1, 1, 1])
    assert ev.t_attn == 18.0 and ev.n_tasks == 16
    # 16 rows over 32 warps: no run leaves the 0.8 x 32 = 25.6 units the rule
    # asks for (run 1 gives 16), so the run stays at 1
    assert PL.reduction_run(pb, prm) == 1


def _check_plan_invariants(pb, prm, ev):
    lim = PL.split_limits(pb, prm, PL.reference_plan(pb, prm))
    T = prm.tile_tokens
    for b, L in enumerate(pb.seq_lens):
        s = ev.splits[b]
        assert 1 <= s <= max(lim[b], PL.reference_plan(pb, prm)[b])
        rng = PL.split_ranges(L, s, T)
        assert rng[0][0] == 0 and rng[-1][1] == L
        for (a0, e0), (a1, e1) in zip(rng, rng[1:]):
            assert e0 == a1 and a0 < e0
        for a, e in rng:
            assert a % T == 0 and (e % T == 0 or e == L)


@pytest.mark.parametrize("seed", range(8))
def test_random_batches_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    L = rng.integers(1, 5000, size=B).tolist()
    n = [1] * B
    if seed % 3 == 0:
        n[0] = min(L[0], int(rng.integers(17, 64)))
    pb = PL.Problem(seq_lens=L, q_lens=n, num_kv_heads=int(rng.integers(1, 4)),
                    rows_per_token=4, n_ext=int(seed % 2))
    prm = PL.Params(slots=int(rng.integers(2, 24)), warps_per_slot=2)
    ev = PL.plan(pb, prm)
    _check_plan_invariants(pb, prm, ev)
    ns = PL.simulate(pb, prm, [1] * B)
    # adopted split plans are at least min_gain below NoSplit
    if any(s > 1 for s in ev.splits):
        assert ev.score <= 0.9 * ns.score
    else:
        assert ev.score == ns.score


def test_task_order_rules():
    prm = PL.Params(slots=4)
    # split decode-only plan: longest first, stable
    pb = PL.Problem(seq_lens=[64 * 5, 64 * 9], q_lens=[1, 1])
    tasks = PL.build_tasks(pb, prm, [1, 2])
    assert [t.n_t for t in tasks] == [5, 5, 4]
    assert [(t.b, t.r) for t in tasks] == [(0, 0), (1, 0), (1, 1)]
    # unsplit: FIFO
    tasks = PL.build_tasks(pb, prm, [1, 1])
    assert [t.b for t in tasks] == [0, 1]
    # mixed batch: chunk request's tasks first, FIFO otherwise
    pb = PL.Problem(seq_lens=[640, 200], q_lens=[1, 20])
    tasks = PL.build_tasks(pb, prm, [2, 1])
    assert [t.b for t in tasks][:20] == [1] * 20 and [t.b for t in tasks][20:] == [0, 0]
    # causal chunk rows see L - n + i + 1 tokens: tiles grow with i
    assert tasks[0].n_t == math.ceil(181 / 64) and tasks[19].n_t == math.ceil(200 / 64)


def test_balanced_plan_hand_examples():
    # tiles [10, 3, 1], one task per split: t = 1 gives 14 tasks, t = 2 gives [5, 2, 1] = 8
    T = 64
    pb = PL.Problem(seq_lens=[10 * T, 3 * T, 1], q_lens=[1, 1, 1])
    prm = PL.Params(tile_tokens=T, slots=4, max_splits=64)
    assert PL.balanced_plan(pb, prm, 14) == [10, 3, 1]
    assert PL.balanced_plan(pb, prm, 8) == [5, 2, 1]
    assert PL.balanced_plan(pb, prm, 7) == [4, 1, 1]      # t = 3: 4 + 1 + 1 = 6
    assert PL.balanced_plan(pb, prm, 3) == [1, 1, 1]
    assert PL.balanced_plan(pb, prm, 2) is None           # NoSplit already has 3 tasks
    prm.max_splits = 3
    assert PL.balanced_plan(pb, prm, 100) == [3, 3, 1]
    # two KV heads and a 2-token request: each split of request 1 is 4 tasks
    pb = PL.Problem(seq_lens=[10 * T, 3 * T], q_lens=[1, 2], num_kv_heads=2, rows_per_token=2)
    prm = PL.Params(tile_tokens=T, slots=4)
    assert PL.balanced_plan(pb, prm, 12) == [4, 1]   # t = 3: 4*2 + 1*4; t = 2 gives 18
    # Figure 8's histories: one wave of 4 CTAs gives (2,1,1), two waves (4,3,1)
    g, pb, prm = fig8()
    assert PL.balanced_plan(pb, prm, 4) == [2, 1, 1]
    assert PL.balanced_plan(pb, prm, 8) == [4, 3, 1]


@pytest.mark.parametrize("seed", range(6))
def test_balanced_plan_is_smallest_budget(seed):
    # the bisection over the tile budget equals a linear scan from t = 1
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 10))
    L = rng.integers(1, 9000, size=B).tolist()
    n = [int(rng.integers(1, 3)) if rng.random() < 0.3 else 1 for _ in range(B)]
    n = [min(a, b) for a, b in zip(n, L)]
    pb = PL.Problem(seq_lens=L, q_lens=n, num_kv_heads=int(rng.integers(1, 4)),
                    rows_per_token=2)
    prm = PL.Params(slots=int(rng.integers(2, 40)), max_splits=int(rng.integers(2, 80)))
    nt = [PL.n_tiles(x, prm.tile_tokens) for x in L]
    per = [q * pb.num_kv_heads for q in n]
    for wave in (prm.slots, 2 * prm.slots, 4 * prm.slots, 1):
        want = None
        for t in range(1, max(nt) + 1):
            c = [max(1, min(math.ceil(a / t), a, prm.max_splits)) for a in nt]
            if sum(s * m for s, m in zip(c, per)) <= wave:
                want = c
                break
        assert PL.balanced_plan(pb, prm, wave) == want


def test_fig8_choice_with_and_without_balanced_candidates():
    # the balanced candidates of Figure 8 ((2,1,1), (4,3,1), ...) all score above 104
    g, pb, prm = fig8()
    for bc in (0, 1):
        prm.balanced_candidates = bc
        assert list(PL.plan(pb, prm, ref=g["reference_plan"]).splits) == g["chosen"]



# ---------------------------------------------------------------------------
# Reference plan (the batch-wide split count standing in for FA3's heuristic)
# ---------------------------------------------------------------------------

def test_reference_plan_hand_scores_on_fig8_histories():
    # Uniform counts u on Figure 8's problem, derived by hand under the model
    # (K = 4, rho = 3/4, delta_attn = delta_red = 4, gamma = 1, one warp per
    # CTA, fused reductions); the 2-tile request is capped at 2 splits.
    #  u = 2 (2,2,2): tasks 100,100,92,92 run at tau 1; at 92 the two 5-tasks
    #    start (k = 4); at 97 they end, the 100-tasks have 3 left at tau 3/4:
    #    t_attn = 99.25. Reductions 4 + 2 = 6: S0 (ready 99.25) on the warp
    #    free at 97 ends 105.25, S1 (ready 92) ends 103, S2 (ready 97) on a
    #    warp free at 99.25 ends 105.25 -> 105.25.
    #  u = 3 (3,3,2): 68,68,68,63 start; at 63 the second 63 starts, at 68
    #    62,5,5; at 73 the 5s end and 53 and 57 work are left at tau 3/4: the
    #    63-task ends at 112.75, the 62-task at 112.75 + 4 * 3/4 = 115.75.
    #    S1's reduction (4 + 3) starts there: 122.75.
    #  u = 4 (4,4,2): 52 x 4 end at 52, 48 x 4 at 100, then 5,5 at tau 3/4:
    #    t_attn 103.75; fused: S2's reduction 4 + 2 from 103.75 -> 109.75;
    #    separate merge launch: S0's and S1's 4 + 4 also wait for 103.75 ->
    #    111.75.
    g, pb, prm = fig8()
    want = {1: ([1, 1, 1], 152.0, 147.0), 2: ([2, 2, 2], 105.25, 99.25),
            3: ([3, 3, 2], 122.75, 115.75), 4: ([4, 4, 2], 109.75, 103.75)}
    for u, (splits, score, t_attn) in want.items():
        assert PL.uniform_plan(pb, prm, u) == splits
        ev = PL.simulate(pb, prm, splits)
        assert (ev.score, ev.t_attn) == (score, t_attn), u
    prm.overlap_reduction = 0
    assert PL.simulate(pb, prm, [4, 4, 2]).score == 111.75
    assert PL.simulate(pb, prm, [2, 2, 2]).score == 105.25
    # the choice over u = 1..max_splits: u = 2 as soon as it is allowed; the
    # largest count is included in the range (max_splits = 2 must reach it)
    for ov in (0, 1):
        prm.overlap_reduction = ov
        for ms, want_plan in ((1, [1, 1, 1]), (2, [2, 2, 2]), (3, [2, 2, 2]), (4, [2, 2, 2])):
            prm.max_splits = ms
            assert PL.reference_plan(pb, prm) == want_plan, (ov, ms)


def test_reference_plan_breaks_score_ties_by_attention_completion():
    # One request of 3 tiles on K = 3 CTAs, rho = 1, delta_attn = 4,
    # delta_red = 2, gamma = 1, fused reductions (hand derivation):
    #  u = 1: one task of 3 + 4 = 7 at tau 1 -> t_attn 7; reduction 2 + 1 -> 10.
    #  u = 2: tasks 6 and 5 -> t_attn 6; the warp of the never-used third CTA
    #         is free from 0, so the reduction 2 + 2 runs 6..10 -> 10.
    #  u = 3: three tasks of 5 at tau 1 -> t_attn 5; reduction 2 + 3 -> 10.
    # Equal scores: the pages' second key, the earlier attention completion,
    # decides (u = 3). Distinct counts always differ in total splits, so the
    # final smaller-u rule can only meet identical plans.
    prm = PL.Params(tile_tokens=64, slots=3, warps_per_slot=1, rho=1.0, delta_attn=4.0,
                    delta_red=2.0, gamma=1.0, max_splits=6, overlap_reduction=1)
    pb = PL.Problem(seq_lens=[3 * 64], q_lens=[1])
    got = [(PL.simulate(pb, prm, [u]).score, PL.simulate(pb, prm, [u]).t_attn) for u in (1, 2, 3)]
    assert got == [(10.0, 7.0), (10.0, 6.0), (10.0, 5.0)]
    assert PL.reference_plan(pb, prm) == [3]
    # Tiles (6, 3) on K = 2, rho = 1, delta_attn = 0, delta_red = 1, gamma = 1:
    #  u = 1: tasks 6 and 3 -> t_attn 6; reductions of 1 + 1 from 6 -> 8.
    #  u = 2: 3,3 then 2,1 -> t_attn 5; S0's reduction 1 + 2 on the warp free
    #         at 4 ends 7, S1's from 5 ends 8 -> 8, with the earlier t_attn.
    prm = PL.Params(tile_tokens=64, slots=2, warps_per_slot=1, rho=1.0, delta_attn=0.0,
                    delta_red=1.0, gamma=1.0, max_splits=2, overlap_reduction=1)
    pb = PL.Problem(seq_lens=[6 * 64, 3 * 64], q_lens=[1, 1])
    assert [(PL.simulate(pb, prm, [u, u]).score, PL.simulate(pb, prm, [u, u]).t_attn)
            for u in (1, 2)] == [(8.0, 6.0), (8.0, 5.0)]
    assert PL.reference_plan(pb, prm) == [2, 2]


# ---------------------------------------------------------------------------
# Reduction runs (LiquidCP appendix A.2: the largest run in {1, h, 2h, 4h,
# min(8h, 32)} that leaves at least 0.8 x (K x W) reduction tasks)
# ---------------------------------------------------------------------------

def test_reduction_run_takes_the_largest_qualifying_run():
    # h = 4 rows per token, 8 one-token requests, K x W = 10 warps (0.8 x 10 =
    # 8 units): run 1 gives 32 units, every run >= 4 gives one unit per
    # request = 8, exactly the threshold, so the largest candidate, 32, wins
    # (a strict ">" or a "smallest run" reading would give 1)
    pb = PL.Problem(seq_lens=[640] * 8, q_lens=[1] * 8, rows_per_token=4)
    assert PL.reduction_run(pb, PL.Params(slots=5, warps_per_slot=2)) == 32
    # 20 warps: the threshold is 16 units; only run 1 (32 units) qualifies
    # (a reversed "at most 0.8 x warps" reading would give 32)
    assert PL.reduction_run(pb, PL.Params(slots=10, warps_per_slot=2)) == 1
    # 3 requests of 16 tokens x 2 heads (32 rows each), 20 warps (16 units):
    # runs 1, 2, 4, 8, 16 give 96, 48, 24, 12, 6 units -> 4
    pb = PL.Problem(seq_lens=[640] * 3, q_lens=[16] * 3, rows_per_token=2)
    assert PL.reduction_run(pb, PL.Params(slots=10, warps_per_slot=2)) == 4
    # ragged: 4 requests of 3 tokens x 3 heads (9 rows): runs 1, 3, 6, 12, 24
    # give 36, 12, 4 x ceil(9/6) = 8, 4, 4 units; 10 warps -> 8 units: run 6
    pb = PL.Problem(seq_lens=[640] * 4, q_lens=[3] * 4, rows_per_token=3)
    assert PL.reduction_run(pb, PL.Params(slots=5, warps_per_slot=2)) == 6
    # h = 128 (MLA heads): the candidates are 1, 128, 256, 512 and min(1024,
    # 32) = 32; 64 decode requests over 256 warps (204.8 units): run 1 gives
    # 8192 units, 32 gives 256, 128 gives 64 -> 32
    pb = PL.Problem(seq_lens=[640] * 64, q_lens=[1] * 64, rows_per_token=128)
    assert PL.reduction_run(pb, PL.Params(slots=64, warps_per_slot=4)) == 32


def test_reduction_units_follow_the_run():
    # 9 rows with run 6: units of 6 and 3 rows, c_red = delta_red + gamma v s
    pb = PL.Problem(seq_lens=[640] * 4, q_lens=[3] * 4, rows_per_token=3, n_ext=1)
    prm = PL.Params(slots=5, warps_per_slot=2, delta_red=2.5, gamma=0.5)
    units = PL.reduction_units(pb, prm, [2, 1, 3, 1])
    assert [b for b, _ in units] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert [c for _, c in units] == [2.5 + 0.5 * 6 * 3, 2.5 + 0.5 * 3 * 3,
                                     2.5 + 0.5 * 6 * 2, 2.5 + 0.5 * 3 * 2,
                                     2.5 + 0.5 * 6 * 4, 2.5 + 0.5 * 3 * 4,
                                     2.5 + 0.5 * 6 * 2, 2.5 + 0.5 * 3 * 2]


# ---------------------------------------------------------------------------
# Decode requests: at most 16 query tokens (LiquidCP appendix A.2)
# ---------------------------------------------------------------------------

def test_decode_boundary_at_16_tokens():
    assert PL.is_decode(16) and not PL.is_decode(17)
    T, K = 64, 4
    prm = PL.Params(tile_tokens=T, slots=K)
    # limits: a 16-token request with >= K tiles is raised to four splits, a
    # 17-token one keeps its reference count; fewer than K tiles: no raise
    pb = PL.Problem(seq_lens=[10 * T, 10 * T, 3 * T], q_lens=[16, 17, 1])
    assert PL.split_limits(pb, prm, [1, 1, 1]) == [4, 1, 1]
    assert PL.split_limits(pb, prm, [2, 7, 3]) == [4, 7, 3]
    # ordering: with 16 tokens the batch is decode-only, so a split plan is
    # longest first; with 17 the batch is mixed: that request's (chunk) tasks
    # go first, FIFO
    pb16 = PL.Problem(seq_lens=[10 * T, 4 * T], q_lens=[1, 16])
    t16 = PL.build_tasks(pb16, prm, [2, 1])
    assert [t.c for t in t16] == sorted([t.c for t in t16], reverse=True)
    assert (t16[0].b, t16[0].r) == (0, 0)          # a 5-tile split leads
    pb17 = PL.Problem(seq_lens=[10 * T, 4 * T], q_lens=[1, 17])
    t17 = PL.build_tasks(pb17, prm, [2, 1])
    assert [t.b for t in t17] == [1] * 17 + [0, 0]
    assert [t.qi for t in t17[:17]] == list(range(17))


# ---------------------------------------------------------------------------
# The pins above must catch plausible mistakes: each planted mistake below
# (patched into the oracle module for the duration of one check) fails one.
# ---------------------------------------------------------------------------

def _run_strict(units, w):
    return units > 0.8 * w


def _run_reversed(units, w):
    return units <= 0.8 * w


def _make_reduction_run(qualifies, smallest=False):
    def reduction_run(pb, prm):
        h = pb.rows_per_token
        warps = prm.slots * prm.warps_per_slot
        cands = [r for r in (1, h, 2 * h, 4 * h, min(8 * h, 32))
                 if qualifies(sum((n * h + r - 1) // r for n in pb.q_lens), warps)]
        if not cands:
            return 1
        return min(cands) if smallest else max(cands)
    return reduction_run


def _ref_plan_no_max(pb, prm):                 # the range stops short of max_splits
    best, best_u = None, 1
    for u in range(1, prm.max_splits):
        ev = PL.simulate(pb, prm, PL.uniform_plan(pb, prm, u))
        if best is None or ev.key() < best.key():
            best, best_u = ev, u
    return PL.uniform_plan(pb, prm, best_u)


def _ref_plan_score_only(pb, prm):             # ties kept by the first count
    best, best_u = None, 1
    for u in range(1, prm.max_splits + 1):
        ev = PL.simulate(pb, prm, PL.uniform_plan(pb, prm, u))
        if best is None or ev.score < best.score:
            best, best_u = ev, u
    return PL.uniform_plan(pb, prm, best_u)


def _uniform_no_cap(pb, prm, u):               # counts not capped by the tiles
    return [max(1, min(u, prm.max_splits)) for _ in pb.seq_lens]


@pytest.mark.parametrize("name,attr,mutant,pin", [
    ("strict threshold", "reduction_run", _make_reduction_run(_run_strict),
     test_reduction_run_takes_the_largest_qualifying_run),
    ("reversed threshold", "reduction_run", _make_reduction_run(_run_reversed),
     test_reduction_run_takes_the_largest_qualifying_run),
    ("smallest run", "reduction_run", _make_reduction_run(lambda u, w: u >= 0.8 * w, smallest=True),
     test_reduction_run_takes_the_largest_qualifying_run),
    ("reference range", "reference_plan", _ref_plan_no_max,
     test_reference_plan_hand_scores_on_fig8_histories),
    ("reference ties", "reference_plan", _ref_plan_score_only,
     test_reference_plan_breaks_score_ties_by_attention_completion),
    ("uncapped counts", "uniform_plan", _uniform_no_cap,
     test_reference_plan_hand_scores_on_fig8_histories),
    ("decode below 16", "is_decode", lambda n: n < 16, test_decode_boundary_at_16_tokens),
    ("decode up to 17", "is_decode", lambda n: n <= 17, test_decode_boundary_at_16_tokens),
])
def test_planted_planner_mistakes_fail_a_pin(monkeypatch, name, attr, mutant, pin):
    monkeypatch.setattr(PL, attr, mutant)
    with pytest.raises((AssertionError, ValueError, ZeroDivisionError, IndexError)):
        pin()


# ---------------------------------------------------------------------------
# Query tiles: one task per (request, KV head, tile of consecutive query
# tokens, split), costed by the KV tiles its last token sees
# ---------------------------------------------------------------------------

def test_query_tiles_hand_example():
    # L = 130 KV tokens, n = 5 causal query tokens, 64-token tiles: token i sees
    # 126 + i keys, i.e. 2, 2, 2, 3, 3 KV tiles (128 keys are exactly two
    # tiles). Tiles of 2 tokens: (0,1), (2,3), (4) -> their last tokens see
    # 127, 129, 130 keys: 2, 3, 3 tiles.
    prm = PL.Params(tile_tokens=64, slots=4, delta_attn=1.0)
    assert PL.query_tiles(5, 2) == [(0, 1), (2, 3), (4, 4)]
    assert PL.query_tiles(5, 8) == [(0, 4)]
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=1)
    assert [t.n_t for t in PL.build_tasks(pb, prm, [1])] == [2, 2, 2, 3, 3]
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=2)
    tasks = PL.build_tasks(pb, prm, [1])
    assert [(t.qi, t.n_t, t.c) for t in tasks] == [(0, 2, 3.0), (1, 3, 4.0), (2, 3, 4.0)]
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=8)
    assert [t.n_t for t in PL.build_tasks(pb, prm, [1])] == [3]
    # two splits of 3 tiles ([0,128), [128,130)): the first split is whole for
    # every tile, the second is empty for the tile whose last token sees 127;
    # split decode-only plans are longest first (cost n_t + 1), stable in FIFO
    # order (tile, KV head, split)
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=2, num_kv_heads=2)
    tasks = PL.build_tasks(pb, prm, [2])
    assert [(t.qi, t.g, t.r, t.n_t) for t in tasks] == [
        (0, 0, 0, 2), (0, 1, 0, 2), (1, 0, 0, 2), (1, 1, 0, 2), (2, 0, 0, 2), (2, 1, 0, 2),
        (1, 0, 1, 1), (1, 1, 1, 1), (2, 0, 1, 1), (2, 1, 1, 1), (0, 0, 1, 0), (0, 1, 1, 0)]
    # non-causal rows all see the whole history
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=2, causal=False)
    assert [t.n_t for t in PL.build_tasks(pb, prm, [1])] == [3, 3, 3]
    # simulation: three tasks of 3, 4, 4 on four slots at tau = rho = 1 -> 4
    pb = PL.Problem(seq_lens=[130], q_lens=[5], query_tile=2)
    prm = PL.Params(tile_tokens=64, slots=4, rho=1.0, delta_attn=1.0, delta_red=0.0, gamma=0.0)
    ev = PL.simulate(pb, prm, [1])
    assert ev.n_tasks == 3 and ev.t_attn == 4.0


def test_query_tiles_in_balanced_plan():
    # tasks of one split = query tiles x KV heads: 5 tokens in tiles of 2 on 2
    # KV heads = 6 tasks per split; tiles of the 10-tile request: t = 5 gives
    # 2 splits (12 tasks), t = 4 gives 3 (18)
    T = 64
    pb = PL.Problem(seq_lens=[10 * T], q_lens=[5], num_kv_heads=2, query_tile=2)
    prm = PL.Params(tile_tokens=T, slots=4)
    assert PL.balanced_plan(pb, prm, 12) == [2]
    assert PL.balanced_plan(pb, prm, 17) == [2]
    assert PL.balanced_plan(pb, prm, 18) == [3]
    assert PL.balanced_plan(pb, prm, 5) is None


def _tiles_by_first_token(n, qt):           # planted: costs from the tile's first token
    return [(a, a) for a in range(0, n, qt)]


def test_planted_query_tile_mistake_fails_a_pin(monkeypatch):
    monkeypatch.setattr(PL, "query_tiles", _tiles_by_first_token)
    with pytest.raises(AssertionError):
        test_query_tiles_hand_example()
