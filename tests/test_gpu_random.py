"""Randomised GPU parity: seeded random shapes (dtype (fp32, bf16, FP8 KV; FP8 MLA rows), group size, head dim,
page size, batch, ragged lengths, chunk rows, external states, planner or
random split counts) for the GQA and MLA paths, each checked element-wise
against the float64 oracle (partial states and merged outputs)."""
import math

import numpy as np
import pytest

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import check_all, spec_of

pytestmark = pytest.mark.gpu


def _lengths(rng, batch, q_lens, cap):
    L = []
    for n in q_lens:
        kind = rng.integers(0, 4)
        if kind == 0:
            x = int(rng.integers(1, 70))            # around one or two tiles
        elif kind == 1:
            x = int(rng.integers(60, 700))
        else:
            x = int(rng.integers(500, cap))
        L.append(max(x, n))
    return L


def _plan(rng, w):
    spec = spec_of(w)
    if rng.integers(0, 2) == 0:
        return skv.plan_splits(w.seq_lens, spec, int(rng.choice([4, 8, 64, 256])), q_lens=w.q_lens,
                               n_ext=w.n_ext)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in w.seq_lens]
    counts = [min(c, 64) for c in counts]
    # 4 CUs gives merge units of several rows (the work-group-per-unit merge)
    return skv.plan_from_counts(w.seq_lens, spec, counts, int(rng.choice([4, 256])), q_lens=w.q_lens,
                                n_ext=w.n_ext)


@pytest.mark.parametrize("seed", range(40))
def test_random_gqa(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = str(rng.choice(["f32", "bf16"]))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8, 16]))   # bf16 8 and 16 run on the matrix cores
    H_kv = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 6))
    q_lens = [int(rng.integers(2, 24)) if rng.random() < 0.2 else 1 for _ in range(batch)]
    seq = _lengths(rng, batch, q_lens, 2500)
    n_ext = int(rng.choice([0, 0, 1, 3, 12, 64]))
    w = wl.build(f"rand-gqa-{seed}", dtype=dtype, mla=False, seq_lens=seq, q_lens=q_lens,
                 num_q_heads=G * H_kv, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D, page_size=P,
                 scale=1.0 / math.sqrt(D), seed=seed, q_scale=float(rng.choice([1.0, 3.0])),
                 causal=True, n_ext=n_ext, ext_lse_center=4.0)
    check_all(w, _plan(rng, w))


@pytest.mark.parametrize("seed", range(20))
def test_random_mla(seed):
    rng = np.random.default_rng(2000 + seed)
    H = int(rng.choice([16, 32, 64, 96, 128]))
    P = int(rng.choice([16, 32, 64]))
    batch = int(rng.integers(1, 5))
    q_lens = [int(rng.integers(2, 12)) if rng.random() < 0.2 else 1 for _ in range(batch)]
    seq = _lengths(rng, batch, q_lens, 2200)
    n_ext = int(rng.choice([0, 0, 2, 16, 64]))
    w = wl.build(f"rand-mla-{seed}", dtype="bf16", mla=True, seq_lens=seq, q_lens=q_lens,
                 num_q_heads=H, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P,
                 scale=wl.MLA_SCALE, seed=seed, value_scale=0.1,
                 q_scale=float(rng.choice([1.0, wl.SHARP_MLA])), causal=True, n_ext=n_ext,
                 ext_lse_center=5.0)
    check_all(w, _plan(rng, w))


@pytest.mark.parametrize("seed", range(16))
def test_random_fp8(seed):
    # FP8 (OCP E4M3) KV with per-(page, KV head) scales: groups of 8 and 16,
    # head dims 64 and 128, page sizes 16-64, ragged lengths, a few chunk rows
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    G = int(rng.choice([8, 16]))
    H_kv = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 6))
    q_lens = [int(rng.integers(2, 24)) if rng.random() < 0.2 else 1 for _ in range(batch)]
    seq = _lengths(rng, batch, q_lens, 2500)
    n_ext = int(rng.choice([0, 0, 1, 3, 12]))
    w = wl.build(f"rand-fp8-{seed}", dtype="fp8", mla=False, seq_lens=seq, q_lens=q_lens,
                 num_q_heads=G * H_kv, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D, page_size=P,
                 scale=1.0 / math.sqrt(D), seed=seed, q_scale=float(rng.choice([1.0, 3.0])),
                 causal=True, n_ext=n_ext, ext_lse_center=4.0)
    check_all(w, _plan(rng, w))


@pytest.mark.parametrize("seed", range(12))
def test_random_fp8_mla(seed):
    # FP8 (OCP E4M3) MLA rows with one scale per page: 16-128 heads, page sizes
    # 16-64, ragged lengths around the 32- and 64-token tiles, chunk rows,
    # external states, planner or random split counts
    rng = np.random.default_rng(4000 + seed)
    H = int(rng.choice([16, 32, 64, 96, 128]))
    P = int(rng.choice([16, 32, 64]))
    batch = int(rng.integers(1, 5))
    q_lens = [int(rng.integers(2, 12)) if rng.random() < 0.2 else 1 for _ in range(batch)]
    seq = _lengths(rng, batch, q_lens, 2200)
    n_ext = int(rng.choice([0, 0, 2, 16, 64]))
    w = wl.build(f"rand-fp8-mla-{seed}", dtype="fp8", mla=True, seq_lens=seq, q_lens=q_lens,
                 num_q_heads=H, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P,
                 scale=wl.MLA_SCALE, seed=seed, value_scale=0.1,
                 q_scale=float(rng.choice([1.0, wl.SHARP_MLA])), causal=True, n_ext=n_ext,
                 ext_lse_center=5.0)
    check_all(w, _plan(rng, w))
