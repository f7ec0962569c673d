"""GPU parity of the one-call path (skv_decode_attn: partial states of every
split into a caller scratch buffer, then the merge) against the two calls it
stands for and against the float64 oracle. Plans built for the fused engine
(overlap_reduction = 1) run attention and merge in one launch: work-groups
publish their tasks through per-request counters and merge once every task of
a request has published; plans built for a merge after attention run two
launches. Both must give the two calls' results bit for bit."""
import math

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, compare, spec_of, tol_for
from oracle import attention as A

pytestmark = pytest.mark.gpu


def _cases():
    yield wl.make(1)
    yield wl.build("wp-bf16-g16", dtype="bf16", mla=False, seq_lens=[1, 700, 4097, 65], num_q_heads=32,
                   num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                   scale=1.0 / math.sqrt(128), seed=11, q_scale=3.0, n_ext=3, ext_lse_center=5.0)
    yield wl.build("wp-bf16-g8-chunk", dtype="bf16", mla=False, seq_lens=[900, 333], q_lens=[1, 20],
                   num_q_heads=16, num_kv_heads=2, head_dim_qk=64, head_dim_v=64, page_size=32,
                   scale=1.0 / 8.0, seed=12)
    yield wl.build("wp-bf16-g16-tiles", dtype="bf16", mla=False, seq_lens=[900, 4000, 64, 333],
                   q_lens=[7, 1, 64, 4], num_q_heads=32, num_kv_heads=2, head_dim_qk=128,
                   head_dim_v=128, page_size=16, scale=1.0 / math.sqrt(128), seed=14, q_scale=3.0,
                   n_ext=1, ext_lse_center=2.0)
    yield wl.build("wp-f32-g8", dtype="f32", mla=False, seq_lens=[2500, 17, 640], num_q_heads=16,
                   num_kv_heads=2, head_dim_qk=64, head_dim_v=64, page_size=32, scale=1.0 / 8.0,
                   seed=15, q_scale=2.0)
    yield wl.build("wp-mla", dtype="bf16", mla=True, seq_lens=[5000, 64, 1500], q_lens=[1, 1, 3],
                   num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                   scale=wl.MLA_SCALE, seed=13, value_scale=0.1, q_scale=wl.SHARP_MLA, n_ext=2,
                   ext_lse_center=8.0)


@pytest.mark.parametrize("w", list(_cases()), ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("overlap", [0, 1], ids=["two-launch", "one-launch"])
def test_one_call_equals_two_calls_and_oracle(w, out_dtype, overlap):
    print(f"[whole] {w.name} {out_dtype} overlap={overlap}", flush=True)
    d = DeviceInputs(w)
    prm = skv.default_params()
    prm.overlap_reduction = overlap
    plan = skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens, n_ext=w.n_ext, params=prm)
    assert plan.info().total_splits > w.batch    # some request is split: the merge has work
    o_part, lse_part = skv.decode_attn_partial(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale)
    o2, l2 = skv.merge_states(o_part, lse_part, plan, d.o_ext, d.lse_ext, out_dtype=out_dtype)
    # scratch filled with NaN first: the path must not read it before writing
    scratch = torch.full((skv.scratch_bytes(plan),), 0xFF, dtype=torch.uint8, device=d.q.device)
    o1, l1 = skv.decode_attn(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale, d.o_ext, d.lse_ext,
                             out_dtype=out_dtype, scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16) if out_dtype == torch.bfloat16 else o1.view(torch.int32),
                       o2.view(torch.int16) if out_dtype == torch.bfloat16 else o2.view(torch.int32))
    assert torch.equal(l1, l2)
    assert plan.read_error_flag() == 0
    # a second call on the same scratch (its counters left by the first)
    o3, l3 = skv.decode_attn(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale, d.o_ext, d.lse_ext,
                             out_dtype=out_dtype, scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.uint8), o1.view(torch.uint8)) and torch.equal(l3, l1)
    # the merged rows against the oracle (bf16 output: the oracle's value
    # rounded once more, so the bound grows by half a bf16 ulp of |O| <= 4)
    tol = dict(tol_for(w))
    if out_dtype == torch.bfloat16:
        tol["abs"] += 2.0 ** -8 * 4
        tol["rel"] = max(tol["rel"], 1e-2)
    o = o1.float().cpu().double().numpy()
    lse = l1.cpu().double().numpy()
    H = w.num_q_heads
    qoff = A.q_offsets(w)
    for b in range(w.batch):
        ids = list(range(int(w.q_lens[b])))
        ref_o, ref_l = A.attention_rows(w, b, ids)
        rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
        if w.n_ext:
            eo = w.o_ext[:, rows].reshape(w.n_ext, len(ids), H, -1).astype(np.float64)
            el = w.lse_ext[:, rows].reshape(w.n_ext, len(ids), H).astype(np.float64)
            ref_o, ref_l = A.merge(np.concatenate([ref_o[None], eo]), np.concatenate([ref_l[None], el]))
        compare(o[rows].reshape(ref_o.shape), ref_o, lse[rows].reshape(ref_l.shape), ref_l, tol,
                f"{w.name} b={b}")
