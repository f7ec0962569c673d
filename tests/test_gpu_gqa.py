"""GPU parity of the GQA paths and of the merge against the float64 oracle:
the vector-ALU kernel (fp32, and bf16 groups below 8 query heads per KV head)
and the matrix-core kernel (bf16 groups of 16, and of 8 with the head columns
filled by copies)."""
import math

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, check_all, compare, run_path, spec_of, tol_for

pytestmark = pytest.mark.gpu


def small(dtype, H_q, H_kv, D, P, seq, q_lens=None, seed=5, q_scale=1.0, causal=True, n_ext=0):
    return wl.build(f"small-{dtype}-{H_q}x{H_kv}-d{D}-p{P}", dtype=dtype, mla=False, seq_lens=seq,
                    q_lens=q_lens, num_q_heads=H_q, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D,
                    page_size=P, scale=1.0 / math.sqrt(D), seed=seed, q_scale=q_scale, causal=causal,
                    n_ext=n_ext, ext_lse_center=4.0)


@pytest.mark.parametrize("sharp", [False, True])
def test_tiny_fp32_fixed_chunks(sharp):
    # batch 2, 4 q heads / 1 KV head, D 64, L = 100 and 257, page 16 permuted,
    # explicit 64-token chunks: 2 + 5 = 7 partial states, then the merge.
    w = wl.make(1, sharp=sharp)
    plan = skv.plan_fixed_chunks(w.seq_lens, spec_of(w), 64)
    assert plan.info().total_splits == 7
    check_all(w, plan)


def test_tiny_fp32_planner_and_explicit_plans():
    w = wl.make(1)
    d = DeviceInputs(w)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256), d)
    for counts in ([1, 1], [2, 5], [2, 3], [1, 4]):
        check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts), d)


RAGGED = [1, 15, 16, 17, 63, 64, 65, 127, 129, 1000, 2049]


@pytest.mark.parametrize("G,D,P", [(1, 64, 16), (2, 128, 32), (4, 64, 64), (8, 128, 16), (16, 64, 16)])
def test_fp32_group_sizes(G, D, P):
    w = small("f32", 2 * G, 2, D, P, RAGGED, seed=G + D + P, q_scale=2.0)
    rng = np.random.default_rng(G)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in RAGGED]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts))


@pytest.mark.parametrize("H_q,H_kv,D,P", [# matrix-core kernel, groups of 8
                                          (64, 8, 128, 16), (8, 1, 64, 32),
                                          # vector-ALU kernel, groups of 1, 4 and 2
                                          (16, 16, 128, 64), (16, 4, 128, 16), (8, 4, 64, 64),
                                          # matrix-core kernel (16 query heads per KV head)
                                          (128, 8, 128, 16), (16, 1, 128, 32), (32, 2, 128, 64),
                                          (16, 1, 64, 16), (64, 4, 64, 64)])
def test_bf16_shapes(H_q, H_kv, D, P):
    w = small("bf16", H_q, H_kv, D, P, RAGGED, seed=H_q + P, q_scale=3.0)
    rng = np.random.default_rng(H_q)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in RAGGED]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts))
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256))


@pytest.mark.parametrize("dtype,G", [("f32", 4), ("bf16", 4), ("bf16", 16)])
def test_causal_chunk_rows(dtype, G):
    # chunked-prefill rows: query token i of n sees L - n + i + 1 tokens
    seq, q = [300, 70, 65, 900], [40, 1, 65, 17]
    w = small(dtype, 2 * G, 2, 64, 16, seq, q_lens=q, seed=11, q_scale=2.0)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [5, 1, 2, 3], q_lens=q))
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=q), check_partials=False)


@pytest.mark.parametrize("dtype,G", [("f32", 8), ("bf16", 8), ("bf16", 16)])
def test_permuted_equals_identity_bitwise(dtype, G):
    w = small(dtype, 2 * G, 2, 128, 16, RAGGED, seed=3)
    wi = wl.identity_layout(w)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [1, 1, 1, 1, 1, 1, 2, 2, 3, 7, 9])
    a = run_path(w, plan)
    b = run_path(wi, plan)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))


def _probe_thresholds(ranges, L, Dv):
    xs = set()
    for a, e in ranges:
        for x in (a - 1, a, a + 1, e - 1, e, e + 1):
            if 0 <= x <= L:
                xs.add(x)
    xs = sorted(xs)[:Dv]
    return xs + [L] * (Dv - len(xs))


@pytest.mark.parametrize("dtype,G,P", [("f32", 4, 16), ("bf16", 4, 32), ("bf16", 16, 16),
                                       ("bf16", 16, 64)])
def test_coverage_probe_recovers_split_ranges(dtype, G, P):
    # q = 0 makes every weight exactly 1: LSE_r = ln(count_r) and, with
    # V[j, d] = 1 if j >= x_d else 0, count_r * O_r[d] = |S_r intersect [x_d, L)|.
    seq = [1000, 2049, 65, 129, 4000]
    w = small(dtype, 2 * G, 2, 64, P, seq, seed=9)
    w.q[...] = 0
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 7, 2, 1, 13])
    ranges = plan.ranges()
    for b, L in enumerate(seq):
        xs = _probe_thresholds(ranges[b], L, w.head_dim_v)
        j = np.arange(L)[:, None]
        vals = (j >= np.array(xs)[None, :]).astype(np.float32)
        vals = np.broadcast_to(vals[:, None, :], (L, w.num_kv_heads, w.head_dim_v))
        if dtype == "bf16":
            vals = wl.f32_to_bf16_bits(np.ascontiguousarray(vals))
        wl.set_logical_values(w, b, vals)
    o_part, lse_part, o, lse = run_path(w, plan)
    e = plan.export()
    H = w.num_q_heads
    for b, L in enumerate(seq):
        xs = np.array(_probe_thresholds(ranges[b], L, w.head_dim_v))
        off = int(e["state_row_offset"][b])
        for r, (a, en) in enumerate(ranges[b]):
            rows = slice(off + r * H, off + (r + 1) * H)
            count = en - a
            assert np.all(np.rint(np.exp(lse_part[rows])) == count)
            want = np.maximum(0, en - np.maximum(a, xs))
            got = np.rint(count * o_part[rows])
            assert np.array_equal(got, np.broadcast_to(want, got.shape)), (b, r)


@pytest.mark.parametrize("q_lens", [None, [1, 5, 3, 1, 17]], ids=["decode", "chunk-rows"])
def test_coverage_probe_token_index_values(q_lens):
    # fp32, q = 0: every visible key gets weight 1. Values V[j, 0] = j and
    # V[j, 1] = j^2 (exact in fp32 for these lengths), the rest 1: a split over
    # [a, e) must give O[0] = mean(j), O[1] = mean(j^2), LSE = ln(e - a), and
    # the merged row of query token i (visible end v) mean(j) and mean(j^2)
    # over [0, v) - a skipped, repeated or shifted token changes both.
    seq = [1000, 2049, 65, 129, 4000]
    w = small("f32", 8, 2, 64, 16, seq, q_lens=q_lens, seed=19)
    w.q[...] = 0
    for b, L in enumerate(seq):
        j = np.arange(L, dtype=np.float64)
        vals = np.ones((L, w.num_kv_heads, w.head_dim_v), np.float32)
        vals[:, :, 0] = j[:, None]
        vals[:, :, 1] = (j * j)[:, None]
        wl.set_logical_values(w, b, vals)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 7, 2, 1, 13], q_lens=w.q_lens)
    o_part, lse_part, o, lse = run_path(w, plan)
    e = plan.export()
    H = w.num_q_heads
    qoff = np.concatenate([[0], np.cumsum(w.q_lens)])
    for b, L in enumerate(seq):
        n = int(w.q_lens[b])
        off = int(e["state_row_offset"][b])
        for r, (a, en) in enumerate(plan.ranges()[b]):
            for i in range(n):
                vis = L - n + i + 1
                lo, hi = a, min(en, vis)
                rows = slice(off + (r * n + i) * H, off + (r * n + i + 1) * H)
                if hi <= lo:
                    assert np.all(np.isneginf(lse_part[rows])) and np.all(o_part[rows] == 0)
                    continue
                jj = np.arange(lo, hi, dtype=np.float64)
                assert np.allclose(lse_part[rows], np.log(hi - lo), rtol=0, atol=1e-5), (b, r, i)
                assert np.allclose(o_part[rows, 0], jj.mean(), rtol=1e-5, atol=0), (b, r, i)
                assert np.allclose(o_part[rows, 1], (jj * jj).mean(), rtol=1e-5, atol=0), (b, r, i)
                assert np.all(o_part[rows, 2:] == 1.0)
        for i in range(n):
            vis = L - n + i + 1
            jj = np.arange(vis, dtype=np.float64)
            rows = slice((int(qoff[b]) + i) * H, (int(qoff[b]) + i + 1) * H)
            assert np.allclose(lse[rows], np.log(vis), rtol=0, atol=1e-5)
            assert np.allclose(o[rows, 0], jj.mean(), rtol=1e-5, atol=0), (b, i)
            assert np.allclose(o[rows, 1], (jj * jj).mean(), rtol=1e-5, atol=0), (b, i)


def test_merge_external_states():
    w = small("f32", 8, 2, 64, 16, [300, 1000, 17], seed=4, n_ext=5)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 4, 1], n_ext=5))
    wb = small("bf16", 16, 2, 128, 32, [300, 1000, 17], seed=4, n_ext=3)
    check_all(wb, skv.plan_splits(wb.seq_lens, spec_of(wb), 256, n_ext=3))


def test_merge_many_states_skip_empty():
    # 12 external states (more than eight per row: the many-state merge path),
    # 128-wide values, a 9-token request so that row runs are ragged; a fifth of
    # the external states are empty (LSE -inf) with NaN vectors, which the merge
    # must not read (the oracle takes an empty state's vector as zero)
    w = small("bf16", 16, 2, 128, 32, [300, 1000, 40], q_lens=[1, 1, 9], seed=6, n_ext=12)
    mask = np.random.default_rng(3).random(w.lse_ext.shape) < 0.2
    w.lse_ext[mask] = -np.inf
    w.o_ext[mask] = np.nan
    d = DeviceInputs(w)
    w.o_ext[mask] = 0.0
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens, n_ext=12), d)


@pytest.mark.parametrize("num_cu", [256, 4])
def test_merge_with_128_states(num_cu):
    # 64 external states and a request in 64 splits: 128 states per row (the
    # most a row can have), so both of each lane's LSE slots are full. num_cu 256
    # gives single-row merge units, 4 gives units of several rows (the
    # work-group-per-unit merge); some external states are empty with NaN
    # vectors (not read; the oracle takes an empty state's vector as zero)
    w = small("bf16", 16, 2, 128, 16, [4200, 900, 70], q_lens=[1, 60, 1], seed=12, n_ext=64)
    mask = np.random.default_rng(7).random(w.lse_ext.shape) < 0.1
    w.lse_ext[mask] = -np.inf
    w.o_ext[mask] = np.nan
    d = DeviceInputs(w)
    w.o_ext[mask] = 0.0
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [64, 14, 2], num_cu, q_lens=w.q_lens, n_ext=64)
    if num_cu == 4:
        assert plan.info().reduction_run >= 8
    check_all(w, plan, d)


def test_bf16_output_rounding():
    w = small("bf16", 16, 2, 128, 16, [500, 77], seed=8)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 2])
    d = DeviceInputs(w)
    o32 = run_path(w, plan, d)[2]
    o16 = run_path(w, plan, d, out_dtype=torch.bfloat16)[2]
    want = wl.f32_to_bf16_bits(o32.astype(np.float32))
    got = wl.f32_to_bf16_bits(o16.astype(np.float32))
    assert np.array_equal(want, got)


@pytest.mark.parametrize("G", [8, 16])
def test_outputs_deterministic(G):
    w = small("bf16", 8 * G, 8, 128, 16, RAGGED, seed=21)
    plan = skv.plan_splits(w.seq_lens, spec_of(w), 256)
    d = DeviceInputs(w)
    a, b = run_path(w, plan, d), run_path(w, plan, d)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))
    assert plan.read_error_flag() == 0


def test_hbm_read_probe_reads_every_word():
    # the probe's per-block XORs combine to the XOR of the whole buffer
    n = (64 << 20) // 4 + 4 * 37   # words; not a multiple of the grid stride
    words = np.random.default_rng(1).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    for blocks in (1, 7, 512):
        out = skv.hbm_read_probe(buf, blocks).cpu().numpy().view(np.uint32)
        assert np.bitwise_xor.reduce(out) == np.bitwise_xor.reduce(words)


def _mix32(x):
    x = np.uint64(x) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16); x = (x * np.uint64(0x7feb352d)) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(15); x = (x * np.uint64(0x846ca68b)) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16)
    return int(x)


def _bf16_pair(h):
    # two bf16 values (sign, exponent 124..127, seven mantissa bits) from a hash
    out = []
    for half in (h & 0xFFFF, h >> 16):
        bits = (half & 0x807F) | ((124 + ((half >> 7) & 3)) << 7)
        out.append(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])
    return out


def test_mfma_probe_products_and_cycles():
    # The probe's first wave recomputed on the host: operand lane layout of the
    # 16x16x32 bf16 product (lane L holds row/column L % 16 and k = 8 (L / 16)
    # .. + 7 of A and B; lane 0's results are rows 0-3 of column 0). With the
    # operands fixed over the trips, each chain is iters * (A_j B_(j%2)).
    iters, blocks, waves = 3, 2, 4
    out = skv.mfma_probe(blocks, waves, iters, "cuda").cpu().numpy()
    assert out.shape == (blocks * waves, 2)
    A = np.zeros((8, 16, 32)); B = np.zeros((2, 32, 16))
    for L in range(64):
        for j in range(8):
            for e in range(4):
                lo, hi = _bf16_pair(_mix32(L * 64 + 4 * j + e))
                A[j, L % 16, 8 * (L // 16) + 2 * e] = lo
                A[j, L % 16, 8 * (L // 16) + 2 * e + 1] = hi
        for j in range(2):
            for e in range(4):
                lo, hi = _bf16_pair(_mix32(0x9E3779B9 ^ (L * 8 + 4 * j + e)))
                B[j, 8 * (L // 16) + 2 * e, L % 16] = lo
                B[j, 8 * (L // 16) + 2 * e + 1, L % 16] = hi
    want = sum(iters * (A[j] @ B[j % 2])[0:4, 0].sum() for j in range(8))
    got = float(out[0, 0:1].view(np.float32)[0])
    assert abs(got - want) <= 1e-4 * max(1.0, abs(want)), (got, want)
    # every wave ran its loop and counted shader cycles (about 17 per product;
    # the bound leaves room for the counter's granularity on 24 products)
    cycles = out[:, 1].astype(np.uint32)
    assert np.all(cycles >= 8 * 8 * iters), cycles


def test_mfma_probe_streaming_waves_read_every_word():
    # with product and streaming waves together, the streaming waves' words
    # combine to the XOR of the buffer over one pass and cancel over two
    n = (16 << 20) // 4 + 4 * 21   # words; not a multiple of the grid stride
    words = np.random.default_rng(2).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    blocks, waves, mw = 5, 8, 3
    for passes, want in ((1, np.bitwise_xor.reduce(words)), (2, np.uint32(0))):
        out = skv.mfma_probe(blocks, waves, 4, "cuda", mfma_waves=mw, buf=buf, passes=passes)
        got = out.cpu().numpy().view(np.uint32).reshape(blocks, waves, 2)
        assert np.bitwise_xor.reduce(got[:, mw:, 0].ravel()) == want, passes
        assert np.all(got[:, :, 1] > 0)
