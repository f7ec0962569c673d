"""The benchmark workloads at full size, in the launch configuration the
benchmark times (critical-wave plan on all CUs, partial attention, merge),
checked against the float64 oracle on sampled output rows (all heads of the
sampled query tokens) and, for one sampled request each, on its partial states.
"""
import sys
import time

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, compare, gpu_partials_of, run_path, spec_of, tol_for
from oracle import attention as A

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[full] {msg}", flush=True)
    sys.stdout.flush()


def bench_plan(w):
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if w.chunk_tokens:
        return skv.plan_fixed_chunks(w.seq_lens, spec_of(w), w.chunk_tokens, num_cu, q_lens=w.q_lens)
    return skv.plan_splits(w.seq_lens, spec_of(w), num_cu, q_lens=w.q_lens, n_ext=w.n_ext)


def check_rows(w, plan, res, samples, partial_req=None):
    """samples: dict request -> list of query-token indices."""
    o_part, lse_part, o, lse = res
    tol = tol_for(w)
    H = w.num_q_heads
    qoff = A.q_offsets(w)
    for b, ids in samples.items():
        t = time.time()
        K, V = A.gather_kv(w, b)
        ro, rl = A.attention_rows(w, b, ids, K=K, V=V)
        if w.n_ext:
            rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
            eo = w.o_ext[:, rows].reshape(w.n_ext, len(ids), H, -1).astype(np.float64)
            el = w.lse_ext[:, rows].reshape(w.n_ext, len(ids), H).astype(np.float64)
            ro, rl = A.merge(np.concatenate([ro[None], eo]), np.concatenate([rl[None], el]))
        rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
        compare(o[rows].reshape(ro.shape), ro, lse[rows].reshape(rl.shape), rl, tol,
                f"{w.name} merged b={b} L={int(w.seq_lens[b])}")
        if b == partial_req:
            po, pl = A.partial_states(w, b, plan.ranges()[b], token_ids=ids, K=K, V=V)
            go, gl = gpu_partials_of(w, plan, o_part, lse_part, b, ids)
            compare(go, po, gl, pl, tol, f"{w.name} partial b={b}")
        log(f"{w.name}: request {b} (L={int(w.seq_lens[b])}, {len(ids)} tokens) ok "
            f"in {time.time() - t:.1f}s")


def value_bound(w) -> float:
    """Largest magnitude any attention output can take: every output is a
    convex combination of value vectors (and, merged, of external outputs),
    so no entry exceeds the largest stored value's magnitude."""
    if w.dtype == "fp8":
        codes = np.abs(A.e4m3_to_f64(np.arange(256, dtype=np.uint8)))
        top = float(np.nanmax(codes))      # 448
        vb = top * float(np.nanmax(w.k_scale if w.v_scale is None else w.v_scale))
    else:
        vals = w.k_pages if w.mla else w.v_pages
        vb = 0.0
        for lo in range(0, vals.shape[0], 2048):   # a few pages at a time (the pool is large)
            blk = vals[lo:lo + 2048]
            if w.mla:
                blk = blk[..., : w.head_dim_v]
            if w.dtype == "bf16":
                # magnitudes of finite bf16 values order like their bit patterns
                mag = blk.view(np.uint16) & np.uint16(0x7FFF)
                mag = mag[mag <= 0x7F80]
                if mag.size:
                    vb = max(vb, float(A.to_f64(np.array([mag.max()], np.uint16), "bf16")[0]))
            else:
                vb = max(vb, float(np.nanmax(np.abs(blk))))
    if w.n_ext:
        vb = max(vb, float(np.abs(w.o_ext).max()))
    return vb


def check_every_row(w, res):
    """Properties of all rows (not only the sampled ones): finite outputs and
    LSEs, and no output entry beyond the largest stored value (a row is a
    convex combination of values)."""
    o_part, lse_part, o, lse = res
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{w.name}: non-finite merged rows"
    vb = value_bound(w)
    assert float(np.abs(o).max()) <= vb * (1 + 1e-2), f"{w.name}: an output exceeds the values' bound {vb}"
    log(f"{w.name}: all {lse.shape[0]} rows finite and within the values' bound")


def run_full(cid, samples_fn, sharp=False, decode_only=False):
    t = time.time()
    w = wl.make(cid, sharp=sharp, decode_only=decode_only)
    log(f"{w.name}: generated in {time.time() - t:.1f}s")
    plan = bench_plan(w)
    d = DeviceInputs(w)
    res = run_path(w, plan, d)
    inf = plan.info()
    log(f"{w.name}: GPU done, {inf.num_tasks} tasks, {inf.total_splits} splits")
    assert plan.read_error_flag() == 0
    check_every_row(w, res)
    samples, partial_req = samples_fn(w)
    check_rows(w, plan, res, samples, partial_req)
    del d
    torch.cuda.empty_cache()


def test_tiny_fp32_full():
    run_full(1, lambda w: ({0: [0], 1: [0]}, 1))


def _spread(w, extra=()):
    L = w.seq_lens
    picks = [int(np.argmax(L)), int(np.argmin(L)), 0, w.batch - 1, *extra]
    return list(dict.fromkeys(picks))


def test_llama405b_gqa_share_full():
    run_full(2, lambda w: ({b: [0] for b in _spread(w, (17,))}, int(np.argmax(w.seq_lens))))


def test_llama405b_gqa_share_sharp_full():
    run_full(2, lambda w: ({b: [0] for b in _spread(w)[:2]}, None), sharp=True)


def test_deepseek_mla_full():
    run_full(3, lambda w: ({b: [0] for b in _spread(w, (40,))}, int(np.argmax(w.seq_lens))))


def test_deepseek_mla_sharp_full():
    run_full(3, lambda w: ({b: [0] for b in _spread(w)[:2]}, None), sharp=True)


def test_skewed_rollout_gqa_full():
    def pick(w):
        longs = [int(b) for b in np.nonzero(w.seq_lens == 262144)[0][:2]]
        shorts = [int(np.argmin(w.seq_lens)), int(np.argmax(np.where(w.seq_lens < 262144, w.seq_lens, 0)))]
        return {b: [0] for b in longs + shorts}, longs[0]
    run_full(4, pick)


def test_million_token_mla_shard_full():
    # 8 decode requests of 1,048,576 tokens plus one 2,048-token chunk over a
    # 65,536-token history, 16 external states merged into every row
    def pick(w):
        return {0: [0], 7: [0], 8: [0, 1, 511, 1023, 1024, 1535, 2046, 2047]}, 8
    run_full(5, pick)


def test_skewed_rollout_gqa_sharp_full():
    def pick(w):
        longs = [int(b) for b in np.nonzero(w.seq_lens == 262144)[0][:1]]
        return {b: [0] for b in longs + [int(np.argmin(w.seq_lens))]}, None
    run_full(4, pick, sharp=True)


def test_million_token_mla_decode_sharp_full():
    run_full(5, lambda w: ({3: [0]}, 3), sharp=True, decode_only=True)


def test_spec_decode_gqa_full():
    # 16 query tokens per request (two query tiles of 8 on a group of 8):
    # tokens at both tiles' edges, on the longest, shortest and two more
    def pick(w):
        return {b: [0, 7, 8, 15] for b in _spread(w, (9,))}, int(np.argmax(w.seq_lens))
    run_full(6, pick)


def test_spec_decode_gqa_sharp_full():
    run_full(6, lambda w: ({b: [0, 5, 15] for b in _spread(w)[:2]}, None), sharp=True)


def test_llama405b_gqa_share_fp8_full():
    # workload 2's shape and lengths over an FP8 E4M3 KV cache
    run_full(7, lambda w: ({b: [0] for b in _spread(w, (17,))}, int(np.argmax(w.seq_lens))))


def test_llama405b_gqa_share_fp8_sharp_full():
    run_full(7, lambda w: ({b: [0] for b in _spread(w)[:2]}, None), sharp=True)


def test_deepseek_mla_fp8_full():
    # workload 3's shape and lengths over FP8 E4M3 latent rows
    run_full(8, lambda w: ({b: [0] for b in _spread(w, (40,))}, int(np.argmax(w.seq_lens))))


def test_deepseek_mla_fp8_sharp_full():
    run_full(8, lambda w: ({b: [0] for b in _spread(w)[:2]}, None), sharp=True)
