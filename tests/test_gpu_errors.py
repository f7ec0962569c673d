"""GPU tests of the device error flag and the NaN states it promises.

An out-of-range page id: the device buffers hold N + 1 pages but the call
passes num_pages = N (a view of the first N pages) and one page-table entry
equal to N. A kernel that failed to check the id would read page N, which is
still inside the allocation, so even a broken check stays in bounds; the test
then sees finite values where NaN is promised. A length mismatch: the device
seq_lens differ from the plan's for one request.

Expected (the header's contract): the flag bit is set, every row of the
states of the tasks that met the error is NaN, the merged rows of the affected
request are NaN, and every other state and merged row matches the oracle."""
import math

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import _dev_tensor, compare, gpu_partials_of, oracle_partials, spec_of, tol_for
from oracle import attention as A

pytestmark = pytest.mark.gpu

SEQ = [300, 1000, 777]
COUNTS = [2, 3, 2]
BAD_REQ, BAD_PAGE = 1, 20          # token 20 * P .. of request 1


def _workload(kind):
    if kind in ("mla", "mla16"):
        return wl.build("err-" + kind, dtype="bf16", mla=True, seq_lens=SEQ, num_q_heads=32,
                        num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                        page_size=32 if kind == "mla" else 16,
                        scale=wl.MLA_SCALE, seed=71, value_scale=0.1, spare_pages=1)
    dtype, H_q, H_kv, D, P = kind
    return wl.build(f"err-{dtype}-{H_q}x{H_kv}", dtype=dtype, mla=False, seq_lens=SEQ,
                    num_q_heads=H_q, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D, page_size=P,
                    scale=1.0 / math.sqrt(D), seed=70 + H_q, spare_pages=1)


KINDS = [("f32", 8, 2, 64, 16),      # vector-ALU kernel
         ("bf16", 32, 2, 128, 16),   # matrix-core kernel, groups of 16
         ("bf16", 16, 2, 128, 32),   # matrix-core kernel, groups of 8
         "mla",                      # one page per 32-token tile
         "mla16"]                    # two pages per tile


def _run(w, plan, k, v, page_table, seq_lens):
    dev = k.device
    q = _dev_tensor(w.q, w.dtype, dev)
    o_part, lse_part = skv.decode_attn_partial(q, k, v, page_table, seq_lens, plan, w.scale)
    o, lse = skv.merge_states(o_part, lse_part, plan)
    flag = plan.read_error_flag(dev)   # synchronises
    return (flag, o_part.cpu().double().numpy(), lse_part.cpu().double().numpy(),
            o.cpu().double().numpy(), lse.cpu().double().numpy())


def _check_rows(w, plan, o_part, lse_part, o, lse, bad_states):
    """bad_states: {request: set of split indices whose states must be NaN};
    requests with any NaN state must have NaN merged rows."""
    tol = tol_for(w)
    H = w.num_q_heads
    ref = oracle_partials(w, plan)
    for b in range(w.batch):
        go, gl = gpu_partials_of(w, plan, o_part, lse_part, b)
        ro, rl = ref[b]
        bad = bad_states.get(b, set())
        for r in range(go.shape[0]):
            if r in bad:
                assert np.isnan(go[r]).all() and np.isnan(gl[r]).all(), f"b={b} split {r} not NaN"
            else:
                compare(go[r], ro[r], gl[r], rl[r], tol, f"{w.name} b={b} split {r}")
        rows = slice(b * H, (b + 1) * H)   # one query token per request
        if bad:
            assert np.isnan(o[rows]).all() and np.isnan(lse[rows]).all(), f"merged b={b} not NaN"
        else:
            ref_o, ref_l = A.attention_rows(w, b, [0])
            compare(o[rows].reshape(ref_o.shape), ref_o, lse[rows].reshape(ref_l.shape), ref_l, tol,
                    f"{w.name} merged b={b}")


@pytest.mark.parametrize("kind", KINDS, ids=lambda k: k if isinstance(k, str) else f"{k[0]}-G{k[1] // k[2]}")
def test_out_of_range_page_id(kind):
    w = _workload(kind)
    print(f"[err] page id case {w.name}", flush=True)
    N = w.num_pages
    dev = torch.device("cuda:0")
    # one more poisoned page after the pool: reachable only through the bad id
    k_np = np.concatenate([w.k_pages, np.full_like(w.k_pages[:1], wl._poison_value(w.dtype))])
    k_full = _dev_tensor(k_np, w.dtype, dev)
    k = k_full[:N]
    if w.mla:
        v = k
    else:
        v_np = np.concatenate([w.v_pages, np.full_like(w.v_pages[:1], wl._poison_value(w.dtype))])
        v = _dev_tensor(v_np, w.dtype, dev)[:N]
    pt = w.page_table.copy()
    pt[BAD_REQ, BAD_PAGE] = N
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), COUNTS)
    flag, o_part, lse_part, o, lse = _run(w, plan, k, v, torch.from_numpy(pt).to(dev),
                                          torch.from_numpy(w.seq_lens).to(dev))
    assert flag == 1, flag
    tok = BAD_PAGE * w.page_size
    bad = {r for r, (lo, hi) in enumerate(plan.ranges()[BAD_REQ]) if lo <= tok < hi}
    assert len(bad) == 1
    _check_rows(w, plan, o_part, lse_part, o, lse, {BAD_REQ: bad})
    # the same call on the intact table: no flag, every row matches
    plan2 = skv.plan_from_counts(w.seq_lens, spec_of(w), COUNTS)
    flag, o_part, lse_part, o, lse = _run(w, plan2, k, v, torch.from_numpy(w.page_table).to(dev),
                                          torch.from_numpy(w.seq_lens).to(dev))
    assert flag == 0
    _check_rows(w, plan2, o_part, lse_part, o, lse, {})


@pytest.mark.parametrize("kind", KINDS, ids=lambda k: k if isinstance(k, str) else f"{k[0]}-G{k[1] // k[2]}")
def test_device_lengths_differ_from_plan(kind):
    w = _workload(kind)
    print(f"[err] length case {w.name}", flush=True)
    dev = torch.device("cuda:0")
    k = _dev_tensor(w.k_pages, w.dtype, dev)
    v = k if w.mla else _dev_tensor(w.v_pages, w.dtype, dev)
    sl = w.seq_lens.copy()
    sl[BAD_REQ] -= 1                       # shorter: the page table still covers it
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), COUNTS)
    flag, o_part, lse_part, o, lse = _run(w, plan, k, v, torch.from_numpy(w.page_table).to(dev),
                                          torch.from_numpy(sl).to(dev))
    assert flag == 2, flag
    _check_rows(w, plan, o_part, lse_part, o, lse, {BAD_REQ: set(range(COUNTS[BAD_REQ]))})


@pytest.mark.parametrize("kind", KINDS, ids=lambda k: k if isinstance(k, str) else f"{k[0]}-G{k[1] // k[2]}")
def test_one_launch_path_errors(kind):
    # the fused engine's launch (a plan built with overlap_reduction = 1): a
    # bad page id in one request and a length mismatch in another; their
    # merged rows are NaN, the third request's match the oracle, both bits set
    w = _workload(kind)
    print(f"[err] one-launch case {w.name}", flush=True)
    dev = torch.device("cuda:0")
    N = w.num_pages
    # as above: the bad id N names a poisoned page that exists in memory but
    # lies outside the num_pages = N view the call is given
    k_np = np.concatenate([w.k_pages, np.full_like(w.k_pages[:1], wl._poison_value(w.dtype))])
    k = _dev_tensor(k_np, w.dtype, dev)[:N]
    if w.mla:
        v = k
    else:
        v_np = np.concatenate([w.v_pages, np.full_like(w.v_pages[:1], wl._poison_value(w.dtype))])
        v = _dev_tensor(v_np, w.dtype, dev)[:N]
    prm = skv.default_params()
    prm.overlap_reduction = 1
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), COUNTS, params=prm)
    pt = w.page_table.copy()
    pt[BAD_REQ, BAD_PAGE] = N
    sl = w.seq_lens.copy()
    sl[2] -= 1
    q = _dev_tensor(w.q, w.dtype, dev)
    o, lse = skv.decode_attn(q, k, v, torch.from_numpy(pt).to(dev), torch.from_numpy(sl).to(dev), plan,
                             w.scale)
    assert plan.read_error_flag(dev) == 3
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    H = w.num_q_heads
    for b in (BAD_REQ, 2):
        assert np.isnan(o[b * H:(b + 1) * H]).all() and np.isnan(lse[b * H:(b + 1) * H]).all()
    ref_o, ref_l = A.attention_rows(w, 0, [0])
    compare(o[:H].reshape(ref_o.shape), ref_o, lse[:H].reshape(ref_l.shape), ref_l, tol_for(w),
            f"{w.name} merged b=0")
