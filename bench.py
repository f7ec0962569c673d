"""Benchmark: decode-attention KV GB/s (% of MI355X HBM peak) and tokens/s, 1 GPU.

One step = one attention layer's pass over one batch: the paged partial
attention over every split of the batch's plan, then the LSE merge of the
partial states (and of external states, when the workload has them). The split
plan is built on the host once per batch and reused by every layer; its own
cost is measured separately and reported as ``plan_ms``. Inputs are resident
in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 60] [--warmup 40] [--workload 2]

Prints one JSON line. ``value`` is KV bytes read by the attention (visible
tokens x bytes per token) divided by the time of a step.
"""
from __future__ import annotations

import argparse
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

KERNEL_FILES = {
    "gqa_mfma": "split_kv_partial_amd/csrc/kernels/gqa_mfma.hip",
    "gqa_valu": "split_kv_partial_amd/csrc/kernels/gqa_valu.hip",
    "mla_mfma": "split_kv_partial_amd/csrc/kernels/mla_mfma.hip",
    "merge": "split_kv_partial_amd/csrc/kernels/merge.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=str, default="2",
                    help="1-5, or 5d for the decode-only part of workload 5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the streaming-read probe of the practical HBM read ceiling")
    ap.add_argument("--plan-param", action="append", default=[], metavar="NAME=VALUE",
                    help="override one field of the planner parameters (repeatable)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run one 1 GiB device-to-device copy (a plain copy of known size "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --traffic-probe` into profiles/counters.json and exit")
    return ap.parse_args()


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
    return "gqa_mfma" if (w.dtype == "bf16" and w.group >= 8) else "gqa_valu"


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
    tot = 0
    for L, n in zip(w.seq_lens.astype(np.int64), w.q_lens.astype(np.int64)):
        if w.causal and n > 1:
            tot += int(n * (L - n) + n * (n + 1) // 2)   # row i sees L - n + i + 1 tokens
        else:
            tot += int(L) * int(n)
    return tot


def attention_flops(w) -> float:
    per_head_token = 2.0 * (w.head_dim_qk + w.head_dim_v)
    return per_head_token * w.num_q_heads * visible_kv_tokens(w)


def cpu_baseline(w, target_s: float) -> dict:
    """The oracle, as it is, on requests of the same batch in order (passes over
    the batch repeat) until about target_s seconds of CPU work, with as many
    BLAS threads as the host grants this process (OMP_NUM_THREADS, at most
    16 and at most the CPU count)."""
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
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
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
    attn = [k for k in fetch if "mla_mfma_kernel" in k or "gqa_mfma_kernel" in k or "gqa_valu_kernel" in k]
    assert copy and attn, (list(fetch), "need the copy probe and an attention kernel")
    kib = COPY_PROBE_BYTES / 1024.0
    cf = max(fetch[copy[0]]) / kib        # the probe is the largest copy
    cw = max(write[copy[0]]) / kib
    k = attn[0]
    f_kib = float(np.median(fetch[k]))
    w_kib = float(np.median(write[k]))
    kern = "mla_mfma" if "mla" in k else ("gqa_mfma" if "gqa_mfma" in k else "gqa_valu")
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


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import split_kv_partial_amd as skv
    import workloads as wl

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    wid = args.workload
    cid = int(wid.rstrip("d"))
    t_gen = time.perf_counter()
    w = wl.make(cid, decode_only=wid.endswith("d"))
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] workload {w.name}: batch {w.batch}, generated in {t_gen:.1f}s", file=sys.stderr,
          flush=True)

    def to_dev(a, bf16):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    bf16 = w.dtype == "bf16"
    q = to_dev(w.q, bf16)
    k = to_dev(w.k_pages, bf16)
    v = k if w.mla else to_dev(w.v_pages, bf16)
    pt = torch.from_numpy(w.page_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    o_ext = None if w.o_ext is None else torch.from_numpy(w.o_ext).to(dev)
    lse_ext = None if w.lse_ext is None else torch.from_numpy(w.lse_ext).to(dev)
    spec = skv.AttnSpec(w.num_q_heads, w.num_kv_heads, w.head_dim_qk, w.head_dim_v, w.page_size,
                        dtype=torch.bfloat16 if bf16 else torch.float32, mla=w.mla, causal=w.causal)
    num_cu = torch.cuda.get_device_properties(dev).multi_processor_count

    plan_params = plan_overrides(args.plan_param)

    # host planner, once per batch (timed on its own, after one untimed call
    # that starts the planner's worker threads, a once-per-process cost)
    plan_times = []
    for it in range(21):
        t = time.perf_counter()
        if w.chunk_tokens:
            plan = skv.plan_fixed_chunks(w.seq_lens, spec, w.chunk_tokens, num_cu, q_lens=w.q_lens)
        else:
            plan = skv.plan_splits(w.seq_lens, spec, num_cu, q_lens=w.q_lens, n_ext=w.n_ext,
                                   params=plan_params)
        if it > 0:
            plan_times.append(time.perf_counter() - t)
    info = plan.info()
    ws = plan.workspace(dev)
    o_part = torch.empty(info.state_rows, w.head_dim_v, dtype=torch.float32, device=dev)
    lse_part = torch.empty(info.state_rows, dtype=torch.float32, device=dev)
    o_out = torch.empty(info.total_rows, w.head_dim_v, dtype=torch.float32, device=dev)
    lse_out = torch.empty(info.total_rows, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if args.traffic_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        skv.decode_attn_partial(q, k, v, pt, sl, plan, w.scale, o_part=o_part, lse_part=lse_part)
        skv.merge_states(o_part, lse_part, plan, o_ext, lse_ext, o_out=o_out, lse_out=lse_out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-launch events on the launch stream (torch's current stream): mark[j]
    # precedes launch j (attention and merge alternate) and also ends launch
    # j - 1, so a step carries two events and the first and last bracket the
    # whole timed region
    mark = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        mark[2 * i].record()
        skv.decode_attn_partial(q, k, v, pt, sl, plan, w.scale, o_part=o_part, lse_part=lse_part)
        mark[2 * i + 1].record()
        skv.merge_states(o_part, lse_part, plan, o_ext, lse_ext, o_out=o_out, lse_out=lse_out)
    mark[2 * args.steps].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = mark[0].elapsed_time(mark[2 * args.steps])
    attn_ms = np.array([mark[2 * i].elapsed_time(mark[2 * i + 1]) for i in range(args.steps)])
    merge_ms = np.array([mark[2 * i + 1].elapsed_time(mark[2 * i + 2]) for i in range(args.steps)])
    ms_per_step = total_ms / args.steps
    flag = plan.read_error_flag(dev)

    kv_tokens = visible_kv_tokens(w)
    kv_bytes = kv_tokens * (w.kv_bytes_per_token() if not w.mla else w.head_dim_qk * 2)
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    tokens = int(w.q_lens.sum())
    kern = kernel_of(w)
    attn_avg = float(attn_ms.mean())
    achieved = kv_bytes / (attn_avg * 1e-3) / 1e9
    traffic = measured_traffic(kern, wid)
    roofline = {"kernel": kern, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "launch_ms_avg": round(attn_avg, 4),
                "algorithmic_bytes_per_launch": int(kv_bytes)}
    if w.mla:
        fl = attention_flops(w)
        roofline["mfma_tflops"] = round(fl / (attn_avg * 1e-3) / 1e12, 1)
        roofline["mfma_frac"] = round(fl / (attn_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim_qk": w.head_dim_qk,
                   "head_dim_v": w.head_dim_v, "page_size": w.page_size,
                   "kv_tokens": int(kv_tokens), "query_tokens": tokens, "n_ext": w.n_ext,
                   "splits": int(info.total_splits), "tasks": int(info.num_tasks)},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "attn_ms": round(attn_avg, 4), "merge_ms": round(float(merge_ms.mean()), 4),
        "attn_ms_p95": round(float(np.percentile(attn_ms, 95)), 4),
        "plan_ms": {"p50": round(1e3 * float(np.median(plan_times)), 3),
                    "p95": round(1e3 * float(np.percentile(plan_times, 95)), 3)},
        "ms_per_step_incl_plan": round(ms_per_step + 1e3 * float(np.median(plan_times)), 4),
        "wall_s_timed": round(t_wall, 4), "device_error_flag": flag,
        "roofline": roofline,
    }
    if not args.no_hbm_probe:
        # a measurement beside the step: if its buffer cannot be had, say so
        # and keep the step's line
        try:
            pr = hbm_probe(dev, num_cu)
            out["hbm_probe"] = pr
            out["frac_of_probe"] = round(gbs / pr["gbs"], 4)
            roofline["frac_of_probe"] = round(achieved / pr["gbs"], 4)
        except (RuntimeError, MemoryError) as e:   # torch reports device OOM as RuntimeError
            out["hbm_probe"] = None
            print(f"[bench] HBM probe skipped: {e}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
