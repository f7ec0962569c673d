"""GPU test of the entry point that allocates nothing (skv_decode_attn_noalloc):
through the C ABI, on two calls in a row (the second with a smaller input),
its output must equal skv_decode_attn's (the same kernels over a caller
scratch buffer) bit for bit and match the float64 oracle; a plan that needs
more scratch than the array holds is refused before any launch."""
import math

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, compare, spec_of, tol_for
from oracle import attention as A

pytestmark = pytest.mark.gpu


def _check_oracle(w, o, lse):
    H = w.num_q_heads
    qoff = A.q_offsets(w)
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    for b in range(w.batch):
        ids = list(range(int(w.q_lens[b])))
        ref_o, ref_l = A.attention_rows(w, b, ids)
        rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
        if w.n_ext:
            eo = w.o_ext[:, rows].reshape(w.n_ext, len(ids), H, -1).astype(np.float64)
            el = w.lse_ext[:, rows].reshape(w.n_ext, len(ids), H).astype(np.float64)
            ref_o, ref_l = A.merge(np.concatenate([ref_o[None], eo]), np.concatenate([ref_l[None], el]))
        compare(o[rows].reshape(ref_o.shape), ref_o, lse[rows].reshape(ref_l.shape), ref_l, tol_for(w),
                f"{w.name} b={b}")


def _one(w):
    d = DeviceInputs(w)
    plan = skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens, n_ext=w.n_ext)
    assert skv.scratch_bytes(plan) <= skv.NOALLOC_SCRATCH_BYTES
    o_ref, l_ref = skv.decode_attn(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale, d.o_ext,
                                   d.lse_ext)
    o, l = skv.decode_attn_noalloc(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale, d.o_ext,
                                   d.lse_ext)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32)), w.name
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32)), w.name
    assert plan.read_error_flag() == 0
    _check_oracle(w, o, l)
    return plan


@pytest.mark.parametrize("family", ["mla", "gqa"])
def test_noalloc_two_calls_second_smaller(family):
    print(f"[noalloc] {family}", flush=True)
    if family == "mla":
        big = wl.build("na-mla-big", dtype="bf16", mla=True, seq_lens=[40000, 9000, 130, 20000],
                       q_lens=[1, 2, 1, 1], num_q_heads=128, num_kv_heads=1, head_dim_qk=576,
                       head_dim_v=512, page_size=64, scale=wl.MLA_SCALE, seed=31, value_scale=0.1,
                       q_scale=wl.SHARP_MLA, n_ext=2, ext_lse_center=9.0)
        small = wl.build("na-mla-small", dtype="bf16", mla=True, seq_lens=[700, 65], num_q_heads=64,
                         num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=32,
                         scale=wl.MLA_SCALE, seed=32, value_scale=0.1)
    else:
        big = wl.build("na-gqa-big", dtype="bf16", mla=False, seq_lens=[30000, 17, 8000, 4100],
                       num_q_heads=128, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=16,
                       scale=1.0 / math.sqrt(128), seed=33, q_scale=3.0)
        small = wl.make(1)
    p1 = _one(big)
    p2 = _one(small)
    assert skv.scratch_bytes(p2) < skv.scratch_bytes(p1)


def test_noalloc_refuses_plans_beyond_its_array():
    # 2048 query tokens x 128 MLA heads x several splits need far more than
    # 128 MiB of partial states: refused on the host, nothing launched
    spec = skv.AttnSpec(128, 1, 576, 512, 64, mla=True)
    plan = skv.plan_fixed_chunks([65536 + 2048], spec, 8192, q_lens=[2048])
    assert skv.scratch_bytes(plan) > skv.NOALLOC_SCRATCH_BYTES
    desc = spec.desc(1, max_pages=1100, num_pages=1100, scale=0.07)
    import ctypes
    st = skv._lib.skv_decode_attn_noalloc(ctypes.byref(desc), 256, 256, 256, 256, 256, plan.handle, 256, 0,
                                          None, None, 256, 0, None, None)
    assert st == -4, st
    assert "scratch" in skv._lib.skv_last_error().decode()
