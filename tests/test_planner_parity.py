"""The library's C++ planner against the reference planner, bit for bit (CPU).

Split counts, split token ranges, the launch order of the attention tasks and
the model scores (as IEEE doubles) must be identical. The LiquidCP Figure 8
example (section 5.2) is also checked through the C ABI.
"""
import json
import os
import struct
import time

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from oracle import planner as PL


def bits(x: float) -> int:
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def reference_for(plan: skv.Plan, spec: skv.AttnSpec, seq, qlen, n_ext=0, params=None, ref=None):
    inf = plan.info()
    p = params or skv.default_params()
    prm = PL.Params(tile_tokens=64, slots=inf.slots, warps_per_slot=inf.warps_per_slot,
                    rho=inf.rho, delta_attn=inf.delta_attn, delta_red=inf.delta_red,
                    gamma=inf.gamma, max_splits=p.max_splits, min_gain=p.min_gain,
                    overlap_reduction=p.overlap_reduction,
                    balanced_candidates=inf.balanced_candidates)
    pb = PL.Problem(seq_lens=[int(x) for x in seq], q_lens=[int(x) for x in qlen],
                    num_kv_heads=spec.num_kv_heads, rows_per_token=spec.num_q_heads, n_ext=n_ext,
                    causal=spec.causal, query_tile=inf.query_tile)
    return pb, prm, PL.plan(pb, prm, ref=ref), PL.simulate(pb, prm, [1] * len(seq))


def assert_same(plan: skv.Plan, pb, prm, ev, ns):
    inf = plan.info()
    e = plan.export()
    assert e["split_counts"].tolist() == list(ev.splits)
    exp_ranges = [r for b, L in enumerate(pb.seq_lens) for r in PL.split_ranges(L, ev.splits[b], 64)]
    assert list(zip(e["split_start"].tolist(), e["split_end"].tolist())) == exp_ranges
    tasks = PL.build_tasks(pb, prm, list(ev.splits))
    assert e["task_order"].tolist() == [[t.b, t.g, t.qi, t.r] for t in tasks]
    assert bits(inf.score) == bits(ev.score)
    assert bits(inf.t_attn) == bits(ev.t_attn)
    assert bits(inf.nosplit_score) == bits(ns.score)
    assert inf.reduction_run == PL.reduction_run(pb, prm)


def test_fig8_through_the_abi():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fig8_critical_wave.json")))
    spec = skv.AttnSpec(1, 1, 64, 64, 16, dtype=torch.float32)
    p = skv.default_params()
    p.use_calibration = 0
    p.balanced_candidates = 0   # the pages' candidate set, as in their example
    p.slots_per_cu, p.warps_per_slot = 1, 1
    p.rho, p.delta_attn, p.delta_red, p.gamma = 0.75, 4.0, 4.0, 1.0
    p.overlap_reduction = 1
    seq = [t * 64 for t in g["histories_tiles"]]
    plan = skv.plan_splits(seq, spec, num_cu=4, params=p, ref_splits=g["reference_plan"])
    inf = plan.info()
    assert plan.export()["split_counts"].tolist() == g["chosen"]
    assert inf.score == g["printed"]["critical-wave (2,2,1)"]
    assert inf.nosplit_score == g["printed"]["NoSplit (1,1,1)"]
    fa3 = skv.plan_from_counts(seq, spec, g["reference_plan"], num_cu=4, params=p)
    assert fa3.info().score == g["printed"]["FA3-derived (3,3,1)"]


SPECS = [
    skv.AttnSpec(128, 8, 128, 128, 16),
    skv.AttnSpec(64, 8, 128, 128, 16),
    skv.AttnSpec(4, 1, 64, 64, 16, dtype=torch.float32),
    skv.AttnSpec(128, 1, 576, 512, 64, mla=True),
]


def kernel_tile(spec: skv.AttnSpec) -> int:
    """Query tokens per task the library's kernel for spec takes by default:
    the bf16 matrix-core GQA kernel fills 128 rows of (token, head); the
    others take one token."""
    G = spec.num_q_heads // spec.num_kv_heads
    if spec.dtype == torch.bfloat16 and not spec.mla and G in (8, 16):
        return 128 // G
    return 1


@pytest.mark.parametrize("seed", range(160))
def test_random_batches_bit_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    spec = SPECS[seed % len(SPECS)]
    B = int(rng.integers(1, 20))
    seq = rng.integers(1, 20000, size=B)
    if seed % 5 == 0:
        seq[0] = int(rng.integers(50000, 300000))
    q = np.ones(B, np.int64)
    if seed % 7 == 3:
        q[-1] = min(int(seq[-1]), int(rng.integers(17, 40)))
    num_cu = int(rng.choice([4, 16, 64, 256]))
    n_ext = int(rng.integers(0, 3))
    p = skv.default_params()
    p.overlap_reduction = int(seed % 2)
    p.max_splits = int(rng.choice([4, 8, 16, 64]))
    if seed % 3 == 0:
        p.use_calibration = 0
        p.rho, p.delta_attn, p.gamma = float(rng.uniform(0.2, 0.9)), float(rng.integers(0, 40)), 0.1
    if seed % 11 == 5:
        p.use_calibration = 0
        p.delta_red, p.gamma = 0.0, 0.0        # zero-cost reductions: ties between warps
    if seed % 8 in (1, 7):
        p.balanced_candidates = 1 if seed % 8 == 1 else 0   # against the kernel's default
    if seed % 4 == 2:
        # several query tokens per request on a bf16 GQA problem, whose kernel
        # groups them in query tiles: its default tile, or a smaller one
        spec = SPECS[(seed // 4) % 2]
        q = np.minimum(seq, rng.integers(1, 40, size=B))
        p.query_tile = int(rng.choice([0, 1, 2, kernel_tile(spec)]))
    plan = skv.plan_splits(seq, spec, num_cu=num_cu, q_lens=q, n_ext=n_ext, params=p)
    assert plan.info().balanced_candidates == (
        p.balanced_candidates if p.balanced_candidates >= 0 else int(spec.mla))
    assert plan.info().query_tile == (p.query_tile or kernel_tile(spec))
    pb, prm, ev, ns = reference_for(plan, spec, seq, q, n_ext, p)
    assert_same(plan, pb, prm, ev, ns)


@pytest.mark.parametrize("chunk", range(10))
def test_small_random_batches_bit_exact(chunk):
    # 1,000 small batches in all (100 per case), C++ = Python bit for bit:
    # 1-6 requests of 1-3,000 tokens, some with several query tokens, every
    # kernel's shape, 1-8 CUs (so that K is small and the search takes many
    # steps), both reduction models, random caps, calibrated or random model
    # parameters, forced query tiles where the kernel runs them
    for seed in range(100 * chunk, 100 * (chunk + 1)):
        rng = np.random.default_rng(50000 + seed)
        spec = SPECS[int(rng.integers(0, len(SPECS)))]
        B = int(rng.integers(1, 7))
        seq = rng.integers(1, 3001, size=B)
        q = np.ones(B, np.int64)
        if rng.random() < 0.3:
            k = int(rng.integers(0, B))
            q[k] = min(int(seq[k]), int(rng.integers(2, 40)))
        p = skv.default_params()
        p.overlap_reduction = int(rng.integers(0, 2))
        p.max_splits = int(rng.choice([2, 4, 8, 16, 64]))
        if rng.random() < 0.5:
            p.use_calibration = 0
            p.rho, p.delta_attn = float(rng.uniform(0.1, 1.0)), float(rng.integers(0, 8))
            p.delta_red, p.gamma = float(rng.uniform(0, 3)), float(rng.uniform(0, 1))
        if kernel_tile(spec) > 1 and rng.random() < 0.3:
            p.query_tile = int(rng.integers(1, kernel_tile(spec) + 1))
        num_cu = int(rng.choice([1, 2, 4, 8]))
        n_ext = int(rng.integers(0, 3))
        plan = skv.plan_splits(seq, spec, num_cu=num_cu, q_lens=q, n_ext=n_ext, params=p)
        pb, prm, ev, ns = reference_for(plan, spec, seq, q, n_ext, p)
        assert_same(plan, pb, prm, ev, ns)


@pytest.mark.parametrize("seed", range(24))
def test_several_chunk_requests_bit_exact(seed):
    # batches with 2-4 chunk requests (more than 16 query tokens) among decode
    # requests, on few CUs so that the search takes many steps: a chunk
    # request's candidate resumes from its own earlier run after other
    # requests (before or after it in the chunk-first queue) have changed
    rng = np.random.default_rng(7000 + seed)
    spec = SPECS[[0, 2, 3][seed % 3]]
    n_chunk = int(rng.integers(2, 5))
    B = n_chunk + int(rng.integers(1, 6))
    seq = rng.integers(200, 6000, size=B)
    q = np.ones(B, np.int64)
    for k in rng.choice(B, size=n_chunk, replace=False):
        q[k] = min(int(seq[k]), int(rng.integers(17, 48)))
    p = skv.default_params()
    p.overlap_reduction = 0
    p.max_splits = int(rng.choice([4, 8, 16]))
    if seed % 2:
        p.use_calibration = 0
        p.rho, p.delta_attn = float(rng.uniform(0.2, 1.0)), float(rng.integers(0, 6))
        p.delta_red, p.gamma = float(rng.uniform(0, 2)), float(rng.uniform(0, 0.5))
    num_cu = int(rng.choice([2, 4, 8, 16]))
    n_ext = int(rng.integers(0, 3))
    plan = skv.plan_splits(seq, spec, num_cu=num_cu, q_lens=q, n_ext=n_ext, params=p)
    pb, prm, ev, ns = reference_for(plan, spec, seq, q, n_ext, p)
    assert_same(plan, pb, prm, ev, ns)


@pytest.mark.parametrize("seed", range(40))
def test_library_reference_plan_is_the_oracles(seed):
    # The library evaluates the uniform split counts of its reference plan
    # lowest score bound first and cuts a run as soon as it cannot beat the
    # best count found so far. Handing it the oracle's reference plan must
    # then change nothing: the same plan, bit for bit, as the one it builds
    # on its own.
    rng = np.random.default_rng(9000 + seed)
    spec = SPECS[seed % len(SPECS)]
    B = int(rng.integers(1, 24))
    seq = rng.integers(1, 40000, size=B)
    q = np.ones(B, np.int64)
    if seed % 3 == 1:
        k = int(rng.integers(0, B))
        q[k] = min(int(seq[k]), int(rng.integers(17, 64)))
    p = skv.default_params()
    p.overlap_reduction = int(seed % 4 == 3)
    p.max_splits = int(rng.choice([8, 16, 64]))
    num_cu = int(rng.choice([8, 64, 256]))
    n_ext = int(rng.integers(0, 3))
    own = skv.plan_splits(seq, spec, num_cu=num_cu, q_lens=q, n_ext=n_ext, params=p)
    pb, prm, _, _ = reference_for(own, spec, seq, q, n_ext, p)
    ref = PL.reference_plan(pb, prm)
    given = skv.plan_splits(seq, spec, num_cu=num_cu, q_lens=q, n_ext=n_ext, params=p, ref_splits=ref)
    a, b = own.export(), given.export()
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    ia, ib = own.info(), given.info()
    assert bits(ia.score) == bits(ib.score) and bits(ia.t_attn) == bits(ib.t_attn)
    # and the reference plan itself scores as the oracle's does
    assert bits(ia.reference_score) == bits(PL.simulate(pb, prm, ref).score)
    assert bits(ib.reference_score) == bits(ia.reference_score)


@pytest.mark.parametrize("cid", [1, 2, 5])
def test_benchmark_workloads_bit_exact(cid):
    # (workloads 3-6 at the default split cap: test_default_cap_large_workloads_bit_exact)
    L, n = wl.config_lengths(cid)
    spec = {1: SPECS[2], 2: SPECS[0], 5: SPECS[3]}[cid]
    n_ext = 16 if cid == 5 else 0
    # the pure-Python reference is slow on the larger batches: workload 5 is
    # also checked with a smaller split cap (same model, search and ordering)
    p = skv.default_params()
    if cid == 5:
        p.max_splits = 16
    t0 = time.time()
    plan = skv.plan_splits(L, spec, num_cu=256, q_lens=n, n_ext=n_ext, params=p)
    pb, prm, ev, ns = reference_for(plan, spec, L, n, n_ext, params=p)
    assert_same(plan, pb, prm, ev, ns)
    assert time.time() - t0 < 120


def _plan_signature(cid):
    L, n = wl.config_lengths(cid)
    spec = {2: SPECS[0], 3: SPECS[3]}[cid]
    p = skv.plan_splits(L, spec, num_cu=256, q_lens=n)
    e = p.export()
    return e["split_counts"].tolist(), e["task_order"].tolist(), bits(p.info().score)


def test_concurrent_planners_agree():
    # planners on several threads share one worker pool; a call that finds it
    # busy runs its simulations itself, with the same result
    import threading
    want = {c: _plan_signature(c) for c in (2, 3)}
    got, errs = [], []

    def work(c):
        try:
            for _ in range(3):
                got.append((c, _plan_signature(c)))
        except Exception as e:   # pragma: no cover - reported below
            errs.append(e)

    th = [threading.Thread(target=work, args=(c,)) for c in (2, 3, 2, 3)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=300)
    assert not errs and len(got) == 12
    for c, sig in got:
        assert sig == want[c]


def test_planner_in_forked_child():
    # a forked child has no pool workers: it must plan on its own thread
    import multiprocessing as mp
    want = _plan_signature(2)
    ctx = mp.get_context("fork")
    with ctx.Pool(1) as pool:
        got = pool.apply_async(_plan_signature, (2,)).get(timeout=120)
    assert got == want


@pytest.mark.parametrize("B", [2048, 4096])
def test_large_skewed_batches(B):
    # thousands of requests with a few of 1M tokens: the C++ planner finishes
    # in seconds and its plan keeps the invariants (the pure-Python reference
    # is too slow for these sizes; the bit-exact tests cover smaller batches)
    rng = np.random.default_rng(B)
    L = rng.integers(1, 40000, size=B)
    L[rng.choice(B, 16, replace=False)] = 1 << 20
    for spec in (SPECS[0], SPECS[3]):
        t0 = time.time()
        plan = skv.plan_splits(L, spec, num_cu=256)
        assert time.time() - t0 < 30
        inf = plan.info()
        e = plan.export()
        counts = e["split_counts"]
        tiles = (L + 63) // 64
        assert np.all(counts >= 1) and np.all(counts <= np.minimum(tiles, 64))
        starts, ends = e["split_start"], e["split_end"]
        off = np.concatenate([[0], np.cumsum(counts)])
        for b in range(B):
            s, en = starts[off[b]:off[b + 1]], ends[off[b]:off[b + 1]]
            assert s[0] == 0 and en[-1] == L[b] and np.all(s[1:] == en[:-1]) and np.all(s < en)
        assert inf.total_splits == counts.sum()
        assert inf.num_tasks == counts.sum() * spec.num_kv_heads
        if inf.split_adopted:
            assert inf.score <= 0.9 * inf.nosplit_score
        else:
            assert np.all(counts == 1)


def _default_cap_case(cid: int) -> None:
    """C++ = Python at the library's default parameters (split cap 64) on a
    benchmark workload: the plans the bench and the full-size GPU tests use."""
    L, n = wl.config_lengths(cid)
    if cid == 4:   # the workload's own request order (a seeded shuffle)
        order = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(wl.SEED_BASE + 4).spawn(8)[1])).permutation(len(L))
        L, n = L[order], n[order]
    spec = {2: SPECS[0], 3: SPECS[3], 4: SPECS[1], 5: SPECS[3], 6: SPECS[1]}[cid]
    n_ext = 16 if cid == 5 else 0
    plan = skv.plan_splits(L, spec, num_cu=256, q_lens=n, n_ext=n_ext)
    assert plan.info().balanced_candidates == int(spec.mla)
    pb, prm, ev, ns = reference_for(plan, spec, L, n, n_ext)
    assert prm.max_splits == 64
    assert_same(plan, pb, prm, ev, ns)


def test_default_cap_benchmark_workload_2_bit_exact():
    _default_cap_case(2)


@pytest.mark.slow
def test_default_cap_large_workloads_bit_exact():
    # the pure-Python reference takes 0.5-2 minutes per workload here, so the
    # four run side by side in child processes
    import subprocess
    import sys
    tests = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests)
    procs = {}
    for cid in (3, 4, 5, 6):
        code = (f"import sys; sys.path[:0] = [{root!r}, {tests!r}]; "
                f"import test_planner_parity as t; t._default_cap_case({cid}); print('ok')")
        procs[cid] = subprocess.Popen([sys.executable, "-c", code], stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE, text=True)
    failed = []
    for cid, p in procs.items():
        try:
            out, err = p.communicate(timeout=900)
        except subprocess.TimeoutExpired:
            p.kill()
            out, err = p.communicate()
            failed.append((cid, "timeout", err[-2000:]))
            continue
        if p.returncode != 0 or out.strip() != "ok":
            failed.append((cid, p.returncode, err[-2000:]))
    assert not failed, failed
