"""GPU parity of multi-token attention tasks (query tiles) against the float64
oracle: the bf16 matrix-core GQA kernel takes tasks of several consecutive
query tokens of one request (up to 128 rows of (token, head)), so that one pass over a split's keys and values serves
every token of the tile. Each case spans several tiles per request, a ragged
last tile, causal rows whose visible ends differ inside a tile, decode
requests of one token beside them, and split boundaries that cut a tile's
keys; the query-tile length is also forced below the kernel's maximum."""
import math

import pytest

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, check_all, spec_of

pytestmark = pytest.mark.gpu


def _tiles_case(G, D, P, causal, seed):
    # q_lens: a decode token, a tile and a ragged tail, exactly two tiles,
    # many tiles, a tile whose rows all see the same keys (non-causal cases)
    qt = 128 // G
    q = [1, qt + 3, 2 * qt, 5 * qt + 1, 3]
    seq = [129, qt + 3 + 70, 2 * qt + 64, 5 * qt + 1 + 1999, 3]
    return wl.build(f"qtiles-G{G}-d{D}-p{P}-{'c' if causal else 'nc'}", dtype="bf16", mla=False,
                    seq_lens=seq, q_lens=q, num_q_heads=2 * G, num_kv_heads=2, head_dim_qk=D,
                    head_dim_v=D, page_size=P, scale=1.0 / math.sqrt(D), seed=seed, q_scale=3.0,
                    causal=causal)


@pytest.mark.parametrize("G,D,P", [(16, 128, 16), (16, 64, 32), (8, 128, 64), (8, 64, 16)])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_query_tiles_default(G, D, P, causal):
    w = _tiles_case(G, D, P, causal, seed=G + D + P + causal)
    print(f"[qtiles] {w.name}", flush=True)
    d = DeviceInputs(w)
    spec = spec_of(w)
    plan = skv.plan_splits(w.seq_lens, spec, 256, q_lens=w.q_lens)
    assert plan.info().query_tile == 128 // G
    check_all(w, plan, d)
    # explicit splits that cut every request's keys in several places
    counts = [max(1, int(L) // 97) for L in w.seq_lens]
    counts = [min(c, (int(L) + 63) // 64) for c, L in zip(counts, w.seq_lens)]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec, counts, q_lens=w.q_lens), d)


@pytest.mark.parametrize("qt", [1, 3, 5])
def test_query_tile_forced_smaller(qt):
    w = _tiles_case(16, 128, 16, True, seed=40 + qt)
    print(f"[qtiles] forced {qt} {w.name}", flush=True)
    prm = skv.default_params()
    prm.query_tile = qt
    plan = skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens, params=prm)
    assert plan.info().query_tile == qt
    check_all(w, plan)


def test_query_tiles_sharp_scores_and_chunk_tail():
    # sharp scores (one key dominates each row) and a request whose tile ends
    # exactly at a page and split boundary
    w = wl.build("qtiles-sharp", dtype="bf16", mla=False, seq_lens=[4096, 64, 1000],
                 q_lens=[16, 8, 11], num_q_heads=32, num_kv_heads=4, head_dim_qk=64, head_dim_v=64,
                 page_size=16, scale=1.0 / 8.0, seed=77, q_scale=8.0)
    print(f"[qtiles] {w.name}", flush=True)
    d = DeviceInputs(w)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens), d)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [64, 1, 3], q_lens=w.q_lens), d)
