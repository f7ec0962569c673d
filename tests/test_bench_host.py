"""Host-side pieces of the benchmark harness (no GPU): the one-GPU guard, the
byte and flop counts of the roofline, and the counter summary with its
source-hash check."""
import csv
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_visible_tokens_and_flops_closed_forms():
    # decode rows see the whole history; a chunk of n rows over L tokens sees
    # L - n + 1 ... L tokens (bottom-right causal)
    w = wl.build("t", dtype="f32", mla=False, seq_lens=[100, 40], q_lens=[1, 8], num_q_heads=4,
                 num_kv_heads=2, head_dim_qk=64, head_dim_v=32, page_size=16, scale=0.125, seed=1)
    vis = 100 + sum(40 - 8 + i + 1 for i in range(8))
    assert bench.visible_kv_tokens(w) == vis
    assert bench.attention_flops(w) == 2.0 * (64 + 32) * 4 * vis


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_counter_summary_scales_by_the_copy_probe(tmp_path, monkeypatch):
    # a private copy of the kernel sources the hash covers
    for f in [bench.KERNEL_FILES["gqa_mfma"], "split_kv_partial_amd/csrc/kernels/device_common.hpp"]:
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    kib = bench.COPY_PROBE_BYTES / 1024
    kern = "void skv::gqa_mfma_kernel<128>(skv::MfmaArgs)"
    _write_counters(tmp_path / "f", [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE", "Counter_Value": 0.5 * kib},
        {"Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
        {"Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1002.0},
        {"Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1001.0}])
    _write_counters(tmp_path / "w", [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE", "Counter_Value": kib},
        {"Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
        {"Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
        {"Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0}])
    os.makedirs(tmp_path / "profiles")
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "2")
    rec = json.load(open(tmp_path / "profiles" / "counters.json"))["gqa_mfma:2"]
    # median 1001 KiB fetched at 0.5 KiB counted per KiB moved, 10 KiB written at 1:1
    assert rec["hbm_bytes_per_launch"] == pytest.approx((1001.0 / 0.5 + 10.0) * 1024.0)
    assert bench.measured_traffic("gqa_mfma", "2") == pytest.approx(rec["hbm_bytes_per_launch"])
    # an edit to the kernel source invalidates the stored figure
    with open(tmp_path / bench.KERNEL_FILES["gqa_mfma"], "a") as fh:
        fh.write("\n// edited\n")
    assert bench.measured_traffic("gqa_mfma", "2") is None
    assert bench.measured_traffic("gqa_valu", "4") is None


def test_plan_param_overrides():
    assert bench.plan_overrides([]) is None
    p = bench.plan_overrides(["balanced_candidates=0", "rho=0.8", "slots_per_cu=4", "use_calibration=0"])
    assert (p.balanced_candidates, p.slots_per_cu, p.use_calibration) == (0, 4, 0)
    assert p.rho == 0.8
    for bad in (["rho"], ["no_such=1"], ["slots_per_cu=2.5"], ["_fields_=1"]):
        with pytest.raises(ValueError):
            bench.plan_overrides(bad)


def test_kv_bytes_count_each_request_once():
    # a chunk of 8 query tokens shares its request's 40-token history: the KV
    # is read once per request, whatever the number of query tokens
    w = wl.build("t", dtype="bf16", mla=False, seq_lens=[100, 40], q_lens=[1, 8], num_q_heads=4,
                 num_kv_heads=2, head_dim_qk=64, head_dim_v=64, page_size=16, scale=0.125, seed=1)
    assert bench.kv_bytes(w) == 140 * 2 * (64 + 64) * 2
    m = wl.build("m", dtype="bf16", mla=True, seq_lens=[100, 40], q_lens=[1, 8], num_q_heads=16,
                 num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=16, scale=0.07, seed=1)
    assert bench.kv_bytes(m) == 140 * 576 * 2          # MLA rows once: the value is part of the row
    # step bytes: KV + queries + states written and read back + outputs
    rows = 9 * 16
    assert bench.step_bytes(m, state_rows=3 * rows) == (140 * 576 * 2 + 9 * 16 * 576 * 2
                                                        + 2 * 3 * rows * 513 * 4 + rows * 513 * 4)


def test_decode_part_of_the_shard_workload():
    w = wl.build("shard", dtype="bf16", mla=True, seq_lens=[300, 200, 500], q_lens=[1, 1, 20],
                 num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                 scale=0.07, seed=3, n_ext=2)
    d = bench.decode_part(w)
    assert d.batch == 2 and d.n_ext == 0 and d.o_ext is None and d.total_q == 2
    assert np.array_equal(d.page_table, w.page_table[:2]) and d.k_pages is w.k_pages
    assert np.array_equal(d.q, w.q[:2]) and np.array_equal(d.seq_lens, [300, 200])


def test_default_run_is_the_headline_plus_every_other_workload():
    a = bench.parse([])
    assert a.workload == "all" and a.steps == 60 and a.warmup == 40 and a.gpus == 1
    assert bench.HEADLINE == "5d" and bench.PER_CONFIG == ("2", "3", "4", "5", "6", "7", "8")
