"""Benchmark: decode-attention KV GB/s (% of MI355X HBM peak) and tokens/s, 1 GPU.

One step = one attention layer's pass over one batch: the paged partial
attention over every split of the batch's plan, then the LSE merge of the
partial states (and of external states, when the workload has them). The split
plan is built on the host once per batch and reused by every layer; its own
cost is measured separately and reported as ``plan_ms``. Inputs are resident
in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 60] [--warmup 40] [--workload all]

Prints one JSON line. The headline is the decode launch of the million-token
MLA shard (8 requests x 1,048,576 KV tokens, 128 heads, 576/512 dims): the
largest single-GPU workload's decode part, the launch the HBM target is set
on. ``value`` is its KV bytes (each request's KV read once) over the median
step time. ``per_config`` holds the same measurement for the other workloads
(Llama-405B-shaped GQA share, DeepSeek-shaped MLA batch, skewed rollout tail,
the whole million-token shard with its 2,048-token chunked-prefill query and
16 external states per row, a speculative-decoding step of 16 query tokens
per request on a GQA group of 8, the Llama-405B-shaped share over an FP8
E4M3 KV cache, and the DeepSeek-shaped MLA batch over an FP8 E4M3 latent
cache), each with its roofline and its CPU oracle baseline.
``--workload N`` runs one workload alone.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores, vendor figure
METRIC = "decode attention KV GB/s (% of MI355X HBM peak) + tokens/s at 1 GPU"
HEADLINE = "5d"
PER_CONFIG = ("2", "3", "4", "5", "6", "7", "8")

KERNEL_FILES = {
    "gqa_mfma": "split_kv_partial_amd/csrc/kernels/gqa_mfma.hip",
    "gqa_valu": "split_kv_partial_amd/csrc/kernels/gqa_valu.hip",
    "mla_mfma": "split_kv_partial_amd/csrc/kernels/mla_mfma.hip",
    "merge": "split_kv_partial_amd/csrc/kernels/merge.hip",
}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=str, default="all",
                    help="all (headline 5d plus 2-8), or one of 1-8 and 5d (the decode "
                         "requests of workload 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the streaming-read probe of the practical HBM read ceiling")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the probe of the sustained dense bf16 matrix rate")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="print the mixed product + HBM stream probe over a range of flop-per-byte "
                         "ratios (one JSON line each) and exit")
    ap.add_argument("--plan-param", action="append", default=[], metavar="NAME=VALUE",
                    help="override one field of the planner parameters (repeatable)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of each oracle sample")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run one 1 GiB device-to-device copy (a plain copy of known size "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --workload W --traffic-probe` into profiles/counters.json and exit")
    return ap.parse_args(argv)


def hbm_probe(dev, num_cu: int, gib: int = 4, reps: int = 10) -> dict:
    """Practical HBM read ceiling: the library's streaming-read probe over a
    `gib` GiB buffer (well past the 256 MB Infinity Cache), the best median
    of `reps` timed launches over four grid sizes (16-128 work-groups per CU:
    more work-groups read faster, 5.9 TB/s at 4 per CU, 7.0 at 64); HIP events
    on the launch stream."""
    import torch
    import split_kv_partial_amd as skv
    nbytes = gib << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.fill_(0x5A5A5A5A)
    best = None
    for blocks in (16 * num_cu, 32 * num_cu, 64 * num_cu, 128 * num_cu):
        out = torch.empty(blocks, dtype=torch.int32, device=dev)
        for _ in range(3):
            skv.hbm_read_probe(buf, blocks, out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for i in range(reps):
            ev[i].record()
            skv.hbm_read_probe(buf, blocks, out)
        ev[reps].record()
        torch.cuda.synchronize()
        ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "bytes": nbytes, "blocks": blocks, "ms": round(ms, 4)}
    del buf
    torch.cuda.synchronize()
    return best


def _timed_probe_runs(launch, seconds: float) -> float:
    """Average launch time (ms) of `launch` run back to back for about
    `seconds`, so that the clock settles under the load; HIP events on the
    launch stream."""
    import time
    import torch
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    t_end = time.time() + seconds
    e0.record()
    while time.time() < t_end:
        for _ in range(5):
            launch()
        n += 5
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def mfma_probe(dev, num_cu: int, iters: int = 32768, seconds: float = 1.0) -> dict:
    """Sustained dense bf16 matrix rate: the library's matrix-core probe (one
    work-group of four waves per CU, so one wave per SIMD, each keeping eight
    independent 16x16x32 product chains busy on pseudo-random operands). The
    per-wave cycle counts over the launch time give the clock the chip ran
    at."""
    import torch
    import split_kv_partial_amd as skv
    waves = 4
    out = torch.empty(num_cu * waves, 2, dtype=torch.int32, device=dev)
    flops = num_cu * waves * iters * 8 * 16384
    ms = _timed_probe_runs(lambda: skv.mfma_probe(num_cu, waves, iters, dev, out), seconds)
    cycles = float(np.median(out[:, 1].cpu().numpy().astype(np.uint32)))
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "launch_ms": round(ms, 4),
            "cycles_per_product": round(cycles / (8 * iters), 3), "est_ghz": round(cycles / (ms * 1e6), 3)}


def mixed_probe(dev, num_cu: int, flop_per_byte: float, gib: int = 4, passes: int = 2,
                seconds: float = 1.0) -> dict:
    """What a launch that does nothing but bf16 products and an HBM stream
    reaches at the given flop-per-byte ratio: the matrix-core probe with four
    product waves and four streaming waves per CU (one of each per SIMD),
    `passes` non-temporal passes over a `gib` GiB buffer of random words and
    as many products as the ratio asks. Both parts run at once, under the
    chip's power and clock management, with no other work."""
    import torch
    import split_kv_partial_amd as skv
    nbytes = gib << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.random_()
    waves, mw = 8, 4
    B = passes * nbytes
    iters = max(1, int(round(flop_per_byte * B / (num_cu * mw * 8 * 16384))))
    F = num_cu * mw * iters * 8 * 16384
    out = torch.empty(num_cu * waves, 2, dtype=torch.int32, device=dev)
    ms = _timed_probe_runs(lambda: skv.mfma_probe(num_cu, waves, iters, dev, out, mfma_waves=mw, buf=buf,
                                                  passes=passes), seconds)
    cyc = out[:, 1].cpu().numpy().astype(np.uint32).reshape(num_cu, waves).astype(np.float64)
    c_mfma, c_stream = float(np.median(cyc[:, :mw])), float(np.median(cyc[:, mw:]))
    del buf
    torch.cuda.synchronize()
    return {"flop_per_byte": round(F / B, 1), "gbs": round(B / (ms * 1e-3) / 1e9, 1),
            "tflops": round(F / (ms * 1e-3) / 1e12, 1), "launch_ms": round(ms, 4), "bytes": B, "flops": F,
            "est_ghz": round(max(c_mfma, c_stream) / (ms * 1e6), 3),
            "longer_part": "products" if c_mfma >= c_stream else "stream"}


def plan_overrides(items):
    """Planner parameters with NAME=VALUE overrides applied (None if there are
    none); integer fields take integral values, unknown names raise."""
    if not items:
        return None
    import split_kv_partial_amd as skv
    p = skv.default_params()
    for item in items:
        name, sep, val = item.partition("=")
        if not sep or name.startswith("_") or name not in dict(type(p)._fields_):
            raise ValueError(f"bad --plan-param {item!r}")
        cur = getattr(p, name)
        if isinstance(cur, int):
            if float(val) != int(float(val)):
                raise ValueError(f"--plan-param {name} takes an integer, got {val!r}")
            setattr(p, name, int(float(val)))
        else:
            setattr(p, name, float(val))
    return p


def kernel_of(w) -> str:
    if w.mla:
        return "mla_mfma"
    return "gqa_mfma" if (w.dtype in ("bf16", "fp8") and w.group >= 8) else "gqa_valu"


def source_hash(kernel: str) -> str:
    files = [KERNEL_FILES[kernel], "split_kv_partial_amd/csrc/kernels/device_common.hpp"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def visible_kv_tokens(w) -> int:
    """Sum over query tokens of the KV tokens each one attends to."""
    tot = 0
    for L, n in zip(w.seq_lens.astype(np.int64), w.q_lens.astype(np.int64)):
        if w.causal and n > 1:
            tot += int(n * (L - n) + n * (n + 1) // 2)   # row i sees L - n + i + 1 tokens
        else:
            tot += int(L) * int(n)
    return tot


def kv_bytes(w) -> int:
    """Algorithmic KV bytes of an attention launch: every request's KV read
    once (a chunk's query tokens share their request's history), at the
    storage's bytes per token (MLA rows once: the value is part of the row;
    FP8: the codes plus the per-page scales)."""
    return int(round(int(w.seq_lens.astype(np.int64).sum()) * w.kv_bytes_per_token()))


def attention_flops(w) -> float:
    per_head_token = 2.0 * (w.head_dim_qk + w.head_dim_v)
    return per_head_token * w.num_q_heads * visible_kv_tokens(w)


def step_bytes(w, state_rows: int) -> int:
    """HBM bytes a whole step must move at the least: the KV once, queries, the
    partial states written and read back, external states, merged outputs."""
    el = 4 if w.dtype == "f32" else 2   # queries are bf16 over an FP8 cache too
    q = w.total_q * w.num_q_heads * w.head_dim_qk * el
    states = state_rows * (w.head_dim_v + 1) * 4
    ext = w.n_ext * w.total_rows * (w.head_dim_v + 1) * 4
    out = w.total_rows * (w.head_dim_v + 1) * 4
    return kv_bytes(w) + q + 2 * states + ext + out


def cpu_baseline(w, target_s: float) -> dict:
    """The oracle, as it is, on requests of the same batch in order (passes over
    the batch repeat) until about target_s seconds of CPU work, with as many
    BLAS threads as the host grants this process (OMP_NUM_THREADS, at most
    16 and at most the CPU count). Rate: KV bytes the oracle's rows attended
    to (per query token) over its time."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    done_tokens, done_bytes, rows, calls = 0, 0, 0, 0
    per_tok = w.kv_bytes_per_token()
    reqs = set()
    t0 = time.perf_counter()
    threads = max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", "16")), os.cpu_count() or 1))
    with threadpool_limits(limits=threads):
        while time.perf_counter() - t0 < target_s:
            for b in range(w.batch):
                n = int(w.q_lens[b])
                ids = list(range(n)) if n <= 4 else [0, n // 2, n - 1]
                A.attention_rows(w, b, ids)
                for i in ids:
                    vis = A.visible_end(w, b, i)
                    done_tokens += vis
                    done_bytes += vis * per_tok
                rows += len(ids) * w.num_q_heads
                reqs.add(b)
                calls += 1
                if time.perf_counter() - t0 >= target_s:
                    break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"float64 oracle attention, {calls} request evaluations over {len(reqs)} "
                      f"of {w.batch} requests ({rows} output rows, {done_tokens} visible KV "
                      f"tokens) of the same workload, numpy with {threads} BLAS threads"}


COPY_PROBE_BYTES = 1 << 30


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str) -> None:
    """HBM bytes per launch of the attention kernel from a FETCH_SIZE pass and a
    WRITE_SIZE pass, each scaled by what the same counter reads for the 1 GiB
    runtime copy (__amd_rocclr_copyBuffer) of the same run."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    attn = [k for k in fetch if any(n in k for n in ("mla_mfma_kernel", "mla_mfma_f8_kernel", "gqa_mfma_kernel",
                                                      "gqa_rows_kernel", "gqa_valu_kernel"))]
    assert copy and attn, (list(fetch), "need the copy probe and an attention kernel")
    kib = COPY_PROBE_BYTES / 1024.0
    cf = max(fetch[copy[0]]) / kib        # the probe is the largest copy
    cw = max(write[copy[0]]) / kib
    k = attn[0]
    f_kib = float(np.median(fetch[k]))
    w_kib = float(np.median(write[k]))
    kern = "mla_mfma" if "mla" in k else ("gqa_valu" if "gqa_valu" in k else "gqa_mfma")
    hbm = (f_kib / cf + w_kib / cw) * 1024.0
    path = os.path.join(ROOT, "profiles", "counters.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    db[f"{kern}:{workload}"] = {
        "source_hash": source_hash(kern), "kernel": k, "fetch_kib_per_launch": f_kib,
        "write_kib_per_launch": w_kib, "copy_fetch_factor": cf, "copy_write_factor": cw,
        "hbm_bytes_per_launch": hbm, "launches": len(fetch[k])}
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print(json.dumps(db[f"{kern}:{workload}"]))


def decode_part(w5):
    """The decode requests of the million-token shard (its first eight), on the
    same KV pool and page table rows: no chunk request, no external states."""
    nd = int(np.sum(w5.q_lens == 1))
    assert np.all(w5.q_lens[:nd] == 1)
    return dataclasses.replace(w5, name=w5.name + "-decode", seq_lens=w5.seq_lens[:nd].copy(),
                               q_lens=w5.q_lens[:nd].copy(), page_table=w5.page_table[:nd].copy(),
                               q=w5.q[:nd], n_ext=0, o_ext=None, lse_ext=None)


def percentile(a, p) -> float:
    return float(np.percentile(np.asarray(a, np.float64), p))


class Runner:
    """Uploads one workload and times steps of it on the current stream."""

    def __init__(self, w, dev, num_cu, plan_params):
        import torch
        import split_kv_partial_amd as skv
        self.w, self.dev = w, dev
        bf16 = w.dtype == "bf16"

        def to_dev(a):
            # bf16 bits (uint16) become bf16; float32 and FP8 codes (uint8) stay as they are
            if a.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.q = to_dev(w.q)
        self.k = to_dev(w.k_pages)
        self.v = self.k if w.mla else to_dev(w.v_pages)
        self.pt = torch.from_numpy(w.page_table).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)
        self.o_ext = None if w.o_ext is None else torch.from_numpy(w.o_ext).to(dev)
        self.lse_ext = None if w.lse_ext is None else torch.from_numpy(w.lse_ext).to(dev)
        self.k_scale = None if w.k_scale is None else torch.from_numpy(w.k_scale).to(dev)
        # FP8 MLA rows: one scale per page for keys and values (the same tensor)
        self.v_scale = (self.k_scale if w.mla else
                        None if w.v_scale is None else torch.from_numpy(w.v_scale).to(dev))
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": skv.FP8}[w.dtype]
        self.spec = skv.AttnSpec(w.num_q_heads, w.num_kv_heads, w.head_dim_qk, w.head_dim_v, w.page_size,
                                 dtype=dt, mla=w.mla, causal=w.causal)
        # host planner, once per batch (timed on its own, after one untimed
        # call that starts the planner's worker threads, a once-per-process cost)
        self.plan_times = []
        for it in range(21):
            t = time.perf_counter()
            if w.chunk_tokens:
                plan = skv.plan_fixed_chunks(w.seq_lens, self.spec, w.chunk_tokens, num_cu, q_lens=w.q_lens)
            else:
                plan = skv.plan_splits(w.seq_lens, self.spec, num_cu, q_lens=w.q_lens, n_ext=w.n_ext,
                                       params=plan_params)
            if it > 0:
                self.plan_times.append(time.perf_counter() - t)
        self.plan = plan
        self.info = plan.info()
        plan.workspace(dev)
        self.o_part = torch.empty(self.info.state_rows, w.head_dim_v, dtype=torch.float32, device=dev)
        self.lse_part = torch.empty(self.info.state_rows, dtype=torch.float32, device=dev)
        self.o_out = torch.empty(self.info.total_rows, w.head_dim_v, dtype=torch.float32, device=dev)
        self.lse_out = torch.empty(self.info.total_rows, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def attention(self):
        import split_kv_partial_amd as skv
        if self.k_scale is not None:
            skv.decode_attn_partial_fp8(self.q, self.k, self.v, self.k_scale, self.v_scale, self.pt, self.sl,
                                        self.plan, self.w.scale, o_part=self.o_part, lse_part=self.lse_part)
        else:
            skv.decode_attn_partial(self.q, self.k, self.v, self.pt, self.sl, self.plan, self.w.scale,
                                    o_part=self.o_part, lse_part=self.lse_part)

    def merge(self):
        import split_kv_partial_amd as skv
        skv.merge_states(self.o_part, self.lse_part, self.plan, self.o_ext, self.lse_ext,
                         o_out=self.o_out, lse_out=self.lse_out)

    def time_steps(self, steps: int, warmup: int) -> dict:
        """W untimed steps, then K timed ones with HIP events on the launch
        stream (torch's current stream, which the library launches on): mark[j]
        precedes launch j (attention and merge alternate) and also ends launch
        j - 1, so the first and last events bracket the whole timed region."""
        import torch
        for _ in range(warmup):
            self.attention()
            self.merge()
        torch.cuda.synchronize()
        mark = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        for i in range(steps):
            mark[2 * i].record()
            self.attention()
            mark[2 * i + 1].record()
            self.merge()
        mark[2 * steps].record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        attn = np.array([mark[2 * i].elapsed_time(mark[2 * i + 1]) for i in range(steps)])
        merge = np.array([mark[2 * i + 1].elapsed_time(mark[2 * i + 2]) for i in range(steps)])
        total = mark[0].elapsed_time(mark[2 * steps])
        return {"attn": attn, "merge": merge, "step": attn + merge, "total_ms": total, "wall_s": t_wall}

    def free(self):
        import torch
        for name in ("q", "k", "v", "pt", "sl", "o_ext", "lse_ext", "o_part", "lse_part", "o_out", "lse_out",
                     "k_scale", "v_scale"):
            setattr(self, name, None)
        self.plan = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def measure(w, key: str, dev, num_cu: int, args, plan_params) -> dict:
    """One workload's line: step times (median, p95, mean), KV GB/s, tokens/s,
    the attention kernel's roofline and, for the chunked-prefill workload, the
    step against max(bytes / HBM peak, flops / matrix peak)."""
    r = Runner(w, dev, num_cu, plan_params)
    t = r.time_steps(args.steps, args.warmup)
    flag = r.plan.read_error_flag(dev)
    info = r.info
    step_med = float(np.median(t["step"]))
    attn_avg = float(t["attn"].mean())
    kvb = kv_bytes(w)
    fl = attention_flops(w)
    tokens = int(w.q_lens.sum())
    kern = kernel_of(w)
    # the launch's bound: the matrix side when its products take longer at the
    # bf16 peak than its KV bytes at the HBM peak (MLA chunk rows, and MLA
    # over an FP8 cache at 484 flop/B)
    mfma_bound = w.mla and fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) > kvb / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        ach = fl / (attn_avg * 1e-3) / 1e12
        roof = {"kernel": kern, "bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "algorithmic_flops_per_launch": fl}
    else:
        ach = kvb / (attn_avg * 1e-3) / 1e9
        roof = {"kernel": kern, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": int(kvb)}
        if w.mla:
            tf = fl / (attn_avg * 1e-3) / 1e12
            roof["mfma_tflops"] = round(tf, 1)
            roof["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    roof["traffic"] = measured_traffic(kern, key)
    roof["launch_ms_avg"] = round(attn_avg, 4)
    sb = step_bytes(w, info.state_rows)
    t_roof = max(sb / (HBM_PEAK_GBS * 1e9), fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    out = {
        "workload": w.name, "key": key,
        "ms_per_step": round(step_med, 4),
        "ms_per_step_p95": round(percentile(t["step"], 95), 4),
        "ms_per_step_mean": round(float(t["step"].mean()), 4),
        "attn_ms": round(float(np.median(t["attn"])), 4),
        "attn_ms_p95": round(percentile(t["attn"], 95), 4),
        "merge_ms": round(float(np.median(t["merge"])), 4),
        "kv_bytes": int(kvb), "kv_gbs": round(kvb / (step_med * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(kvb / (step_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(tokens / (step_med * 1e-3), 1),
        "step_roofline": {"bytes": int(sb), "flops": fl, "roofline_ms": round(t_roof, 4),
                          "frac": round(t_roof / step_med, 4)},
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim_qk": w.head_dim_qk,
                   "head_dim_v": w.head_dim_v, "page_size": w.page_size,
                   "kv_tokens": int(w.seq_lens.astype(np.int64).sum()), "query_tokens": tokens,
                   "n_ext": w.n_ext, "splits": int(info.total_splits), "tasks": int(info.num_tasks)},
        "plan_ms": {"p50": round(1e3 * float(np.median(r.plan_times)), 3),
                    "p95": round(1e3 * percentile(r.plan_times, 95), 3)},
        "device_error_flag": flag, "roofline": roof,
        "_total_ms": t["total_ms"], "_wall_s": t["wall_s"],
    }
    if np.any(w.q_lens > 1):
        dec = int(np.sum(w.q_lens[w.q_lens == 1]))
        out["decode_tokens_per_s"] = round(dec / (step_med * 1e-3), 1)
        out["prefill_tokens_per_s"] = round((tokens - dec) / (step_med * 1e-3), 1)
    r.free()
    return out


def load(key: str, cache: dict):
    """Workload `key` (1-8, or 5d for the decode part of 5), generated once."""
    import workloads as wl
    if key == "5d":
        return decode_part(load("5", cache))
    if key not in cache:
        t = time.perf_counter()
        cache[key] = wl.make(int(key))
        print(f"[bench] workload {cache[key].name}: batch {cache[key].batch}, generated in "
              f"{time.perf_counter() - t:.1f}s", file=sys.stderr, flush=True)
    return cache[key]


def main(argv=None):
    args = parse(argv)
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import split_kv_partial_amd as skv  # noqa: F401  (fails loudly without the built library)

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    num_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    if args.probe_sweep:
        print(json.dumps({"probe": "hbm", **hbm_probe(dev, num_cu)}), flush=True)
        print(json.dumps({"probe": "mfma", **mfma_probe(dev, num_cu)}), flush=True)
        for r in (32, 64, 128, 192, 242, 320, 512, 1024):
            print(json.dumps({"probe": "mixed", **mixed_probe(dev, num_cu, float(r))}), flush=True)
        return
    plan_params = plan_overrides(args.plan_param)
    head_key = HEADLINE if args.workload == "all" else args.workload
    rest = PER_CONFIG if args.workload == "all" else ()
    cache = {}
    if args.traffic_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head_w = load(head_key, cache)
    head = measure(head_w, head_key, dev, num_cu, args, plan_params)
    print(f"[bench] {head_w.name}: {head['ms_per_step']} ms per step", file=sys.stderr, flush=True)
    per = {}
    for key in rest:
        w = load(key, cache)
        per[key] = measure(w, key, dev, num_cu, args, plan_params)
        print(f"[bench] {w.name}: {per[key]['ms_per_step']} ms per step", file=sys.stderr, flush=True)

    probe = None
    if not args.no_hbm_probe:
        # a measurement beside the steps: if its buffer cannot be had, say so
        # and keep the line
        try:
            probe = hbm_probe(dev, num_cu)
        except (RuntimeError, MemoryError) as e:   # torch reports device OOM as RuntimeError
            print(f"[bench] HBM probe skipped: {e}", file=sys.stderr, flush=True)
    mprobe = xprobe = None
    if not args.no_mfma_probe:
        mprobe = mfma_probe(dev, num_cu)
        # For launches with matrix-side work (MLA rows, query tiles: 64 flop
        # per KV byte or more), the probe with products and a KV stream in the
        # launch's own proportion and nothing else: what the chip reaches there.
        probes = {}
        for key, m in [(head_key, head), *per.items()]:
            w = load(key, cache)
            r = attention_flops(w) / kv_bytes(w)
            if r < 64:
                continue
            rk = round(r)
            if rk not in probes:
                try:
                    probes[rk] = mixed_probe(dev, num_cu, r)
                except (RuntimeError, MemoryError) as e:
                    print(f"[bench] mixed probe skipped: {e}", file=sys.stderr, flush=True)
                    probes[rk] = None
            x = probes[rk]
            if not x:
                continue
            roof = m["roofline"]
            roof["mixed_probe"] = {k: x[k] for k in ("flop_per_byte", "gbs", "tflops", "est_ghz")}
            ref = x["gbs"] if roof["unit"] == "GB/s" else x["tflops"]
            roof["frac_of_mixed_probe"] = round(roof["achieved"] / ref, 4)
            if key == head_key:
                xprobe = x
    for m in [head, *per.values()]:
        if probe:
            m["frac_of_probe"] = round(m["kv_gbs"] / probe["gbs"], 4)
            if m["roofline"]["unit"] == "GB/s":
                m["roofline"]["frac_of_probe"] = round(m["roofline"]["achieved"] / probe["gbs"], 4)
        if mprobe:
            r = m["roofline"]
            tf = r["achieved"] if r["unit"] == "TFLOP/s" else r.get("mfma_tflops")
            if tf is not None:
                r["mfma_frac_of_probe"] = round(tf / mprobe["tflops"], 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        head["cpu_baseline"] = cpu_baseline(head_w, args.cpu_seconds)
        for key in rest:
            per[key]["cpu_baseline"] = cpu_baseline(load(key, cache), args.cpu_seconds)

    total_ms, wall = head.pop("_total_ms"), head.pop("_wall_s")
    for m in per.values():
        m.pop("_total_ms"), m.pop("_wall_s")
    out = {
        "metric": METRIC, "value": head["kv_gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "ms_per_step_p95": head["ms_per_step_p95"], "ms_per_step_mean": head["ms_per_step_mean"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head_w.dtype, "data": "synthetic",
        "config": head["config"],
        "hbm_frac_of_peak": head["hbm_frac_of_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "attn_ms": head["attn_ms"], "attn_ms_p95": head["attn_ms_p95"], "merge_ms": head["merge_ms"],
        "plan_ms": head["plan_ms"],
        "ms_per_step_incl_plan": round(head["ms_per_step"] + head["plan_ms"]["p50"], 4),
        "timed_region_ms": round(total_ms, 3), "wall_s_timed": round(wall, 4),
        "device_error_flag": head["device_error_flag"],
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
    }
    if probe:
        out["hbm_probe"] = probe
        out["frac_of_probe"] = head["frac_of_probe"]
    if mprobe:
        out["mfma_probe"] = mprobe
    if xprobe:
        out["mixed_probe"] = xprobe
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if per:
        out["per_config"] = per
    print(json.dumps(out))


if __name__ == "__main__":
    main()
