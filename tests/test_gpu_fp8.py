"""GPU parity of the FP8 (OCP E4M3) KV cache path against the float64 oracle,
which decodes every code from the format's definition and multiplies it by its
(page, KV head) block's scale. The kernels are the matrix-core GQA kernel
(groups of 16 and of 8, head dims 64 and 128) reading one byte per element, and
the MLA kernel over FP8 latent rows with one scale per page."""
import math

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, _dev_tensor, check_all, compare, run_path, spec_of, tol_for
from oracle import attention as A

pytestmark = pytest.mark.gpu

RAGGED = [1, 15, 16, 17, 63, 64, 65, 127, 129, 1000, 2049]


def fp8_case(H_q, H_kv, D, P, seq, q_lens=None, seed=5, q_scale=1.0, n_ext=0, causal=True):
    return wl.build(f"fp8-{H_q}x{H_kv}-d{D}-p{P}", dtype="fp8", mla=False, seq_lens=seq, q_lens=q_lens,
                    num_q_heads=H_q, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D, page_size=P,
                    scale=1.0 / math.sqrt(D), seed=seed, q_scale=q_scale, n_ext=n_ext,
                    ext_lse_center=4.0, causal=causal)


@pytest.mark.parametrize("H_q,H_kv,D,P", [(32, 2, 128, 16), (16, 1, 64, 32), (16, 2, 128, 64),
                                          (64, 8, 64, 16), (128, 8, 128, 16)])
def test_fp8_shapes(H_q, H_kv, D, P):
    w = fp8_case(H_q, H_kv, D, P, RAGGED, seed=H_q + D + P, q_scale=3.0)
    print(f"[fp8] {w.name}", flush=True)
    d = DeviceInputs(w)
    rng = np.random.default_rng(H_q + P)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in RAGGED]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts), d)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256), d)


def test_fp8_chunk_rows_and_external_states():
    # several query tokens per request (one task per token), causal rows, and
    # external states merged into every row
    w = fp8_case(32, 2, 128, 16, [300, 70, 65, 900], q_lens=[40, 1, 65, 17], seed=11, q_scale=2.0,
                 n_ext=3)
    print(f"[fp8] {w.name} chunk rows", flush=True)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [5, 1, 2, 3], q_lens=w.q_lens, n_ext=3)
    assert plan.info().query_tile == 1
    check_all(w, plan)


def test_fp8_sharp_scores():
    w = fp8_case(16, 2, 64, 16, [4096, 33, 700], seed=21, q_scale=8.0)
    print(f"[fp8] {w.name} sharp", flush=True)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [17, 1, 4]))


def test_fp8_permuted_equals_identity_bitwise():
    w = fp8_case(32, 2, 128, 16, RAGGED, seed=3)
    wi = wl.identity_layout(w)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [1, 1, 1, 1, 1, 1, 2, 2, 3, 7, 9])
    a = run_path(w, plan)
    b = run_path(wi, plan)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_fp8_out_of_range_page_and_flag():
    w = fp8_case(32, 2, 128, 16, [300, 1000, 777], seed=70, n_ext=0)
    print(f"[fp8] {w.name} bad page", flush=True)
    N = w.num_pages
    dev = torch.device("cuda:0")
    # one more poisoned page after the pool, reachable only through the bad id
    k = _dev_tensor(np.concatenate([w.k_pages, np.full_like(w.k_pages[:1], wl.FP8_NAN)]), "fp8", dev)[:N]
    v = _dev_tensor(np.concatenate([w.v_pages, np.full_like(w.v_pages[:1], wl.FP8_NAN)]), "fp8", dev)[:N]
    ks = torch.from_numpy(w.k_scale).to(dev)
    vs = torch.from_numpy(w.v_scale).to(dev)
    pt = w.page_table.copy()
    pt[1, 20] = N
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 3, 2])
    q = _dev_tensor(w.q, "fp8", dev)
    o_part, lse_part = skv.decode_attn_partial_fp8(q, k, v, ks, vs, torch.from_numpy(pt).to(dev),
                                                   torch.from_numpy(w.seq_lens).to(dev), plan, w.scale)
    o, lse = skv.merge_states(o_part, lse_part, plan)
    assert plan.read_error_flag(dev) == 1
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    H = w.num_q_heads
    assert np.isnan(o[H:2 * H]).all() and np.isnan(lse[H:2 * H]).all()
    for b in (0, 2):
        ro, rl = A.attention_rows(w, b, [0])
        compare(o[b * H:(b + 1) * H].reshape(ro.shape), ro, lse[b * H:(b + 1) * H].reshape(rl.shape), rl,
                tol_for(w), f"{w.name} b={b}")


# ---- FP8 MLA latent rows ----

MLA_RAGGED = [1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 1000, 2049]


def fp8_mla(seq, q_lens=None, H=128, P=64, seed=13, q_scale=1.0, causal=True, n_ext=0):
    return wl.build(f"fp8-mla-h{H}-p{P}", dtype="fp8", mla=True, seq_lens=seq, q_lens=q_lens,
                    num_q_heads=H, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P,
                    scale=wl.MLA_SCALE, seed=seed, value_scale=0.1, q_scale=q_scale, causal=causal,
                    n_ext=n_ext, ext_lse_center=5.0)


@pytest.mark.parametrize("sharp", [False, True])
@pytest.mark.parametrize("P", [64, 32, 16])
def test_fp8_mla_ragged(sharp, P):
    # lengths around the 32-token compute tiles and the 64-token FP8 tiles
    w = fp8_mla(MLA_RAGGED, P=P, q_scale=wl.SHARP_MLA if sharp else 1.0, seed=P + sharp)
    print(f"[fp8] {w.name} sharp={sharp}", flush=True)
    d = DeviceInputs(w)
    rng = np.random.default_rng(P + 7)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in MLA_RAGGED]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts), d)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256), d)


@pytest.mark.parametrize("H", [16, 64])
def test_fp8_mla_fewer_heads(H):
    w = fp8_mla([100, 700, 64], H=H, seed=H, q_scale=wl.SHARP_MLA)
    print(f"[fp8] {w.name}", flush=True)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256))


def test_fp8_mla_chunk_rows_and_external_states():
    w = fp8_mla([540, 333, 70], q_lens=[40, 1, 3], seed=3, q_scale=wl.SHARP_MLA, n_ext=4)
    print(f"[fp8] {w.name} chunk rows", flush=True)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 2, 2], q_lens=w.q_lens, n_ext=4))


def test_fp8_mla_permuted_equals_identity_bitwise():
    w = fp8_mla(MLA_RAGGED, seed=5)
    wi = wl.identity_layout(w)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [1] * 6 + [2, 2, 2, 2, 3, 3, 5, 9])
    for x, y in zip(run_path(w, plan), run_path(wi, plan)):
        assert np.array_equal(x, y, equal_nan=True)


def _boost_rope(w, b, j, f):
    """Multiply the decoded rope keys of the page holding token j of request b
    by f, keeping its values: the page's scale times f, its 512 latent codes
    re-encoded from their values divided by f (PyTorch's E4M3 conversion)."""
    pid, _ = wl.physical_slot(w, b, j)
    lat = torch.from_numpy(np.ascontiguousarray(w.k_pages[pid, :, :512])).view(torch.float8_e4m3fn).float()
    w.k_pages[pid, :, :512] = (lat / f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w.k_scale[pid, 0] *= np.float32(f)


@pytest.mark.parametrize("P", [64, 16])
def test_fp8_mla_large_page_scale_restarts(P):
    # late pages whose rope keys decode a hundredfold larger (page scale x100,
    # latent codes /100): their scores exceed the first tile's by far more than
    # 64 (log2 units), so the split runs a second pass from the first pass's
    # maxima; the values keep their size (the weights enter P*V as one bf16
    # term, whose rounding scales with the values)
    w = fp8_mla([3000, 1500, 97], P=P, seed=31, q_scale=wl.SHARP_MLA)
    for b, j in ((0, 2900), (1, 1400), (2, 96)):
        _boost_rope(w, b, j, 100.0)
    print(f"[fp8] {w.name} scaled pages", flush=True)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 1, 1]))


def test_fp8_mla_out_of_range_page_and_flag():
    w = fp8_mla([300, 1000, 777], seed=70)
    print(f"[fp8] {w.name} bad page", flush=True)
    N = w.num_pages
    dev = torch.device("cuda:0")
    # one more poisoned page after the pool, reachable only through the bad id
    kv = _dev_tensor(np.concatenate([w.k_pages, np.full_like(w.k_pages[:1], wl.FP8_NAN)]), "fp8", dev)[:N]
    ks = torch.from_numpy(np.concatenate([w.k_scale, np.full_like(w.k_scale[:1], np.nan)])).to(dev)[:N]
    pt = w.page_table.copy()
    pt[1, 5] = N
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 3, 2])
    q = _dev_tensor(w.q, "fp8", dev)
    o_part, lse_part = skv.decode_attn_partial_fp8(q, kv, kv, ks, ks, torch.from_numpy(pt).to(dev),
                                                   torch.from_numpy(w.seq_lens).to(dev), plan, w.scale)
    o, lse = skv.merge_states(o_part, lse_part, plan)
    assert plan.read_error_flag(dev) == 1
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    H = w.num_q_heads
    assert np.isnan(o[H:2 * H]).all() and np.isnan(lse[H:2 * H]).all()
    for b in (0, 2):
        ro, rl = A.attention_rows(w, b, [0])
        compare(o[b * H:(b + 1) * H].reshape(ro.shape), ro, lse[b * H:(b + 1) * H].reshape(rl.shape), rl,
                tol_for(w), f"{w.name} b={b}")


@pytest.mark.parametrize("mla", [False, True], ids=["gqa", "mla"])
def test_fp8_device_lengths_differ_from_plan(mla):
    # a request's device length one short of the plan's: its tasks read no KV
    # and write NaN states (flag bit 1, value 2); the other requests are exact
    w = fp8_mla([300, 1000, 777], seed=72) if mla else fp8_case(32, 2, 128, 16, [300, 1000, 777], seed=72)
    print(f"[fp8] {w.name} device lengths", flush=True)
    dev = torch.device("cuda:0")
    d = DeviceInputs(w)
    sl = w.seq_lens.copy()
    sl[1] -= 1
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 3, 2])
    o_part, lse_part = skv.decode_attn_partial_fp8(d.q, d.k, d.v, d.k_scale, d.v_scale, d.page_table,
                                                   torch.from_numpy(sl).to(dev), plan, w.scale)
    o, lse = skv.merge_states(o_part, lse_part, plan)
    assert plan.read_error_flag(dev) == 2
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    H = w.num_q_heads
    assert np.isnan(o[H:2 * H]).all() and np.isnan(lse[H:2 * H]).all()
    for b in (0, 2):
        ro, rl = A.attention_rows(w, b, [0])
        compare(o[b * H:(b + 1) * H].reshape(ro.shape), ro, lse[b * H:(b + 1) * H].reshape(rl.shape), rl,
                tol_for(w), f"{w.name} b={b}")
