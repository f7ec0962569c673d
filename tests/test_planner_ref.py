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
    # the run for 16 rows over 32 warps: only run 1 leaves >= 25.6 units -> 16 units
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
