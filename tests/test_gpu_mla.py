"""GPU parity of the MLA path (576-wide latent rows, value = first 512 entries,
up to 128 heads) against the float64 oracle."""
import math

import numpy as np
import pytest

import split_kv_partial_amd as skv
import workloads as wl
from gpu_common import DeviceInputs, check_all, run_path, spec_of

pytestmark = pytest.mark.gpu


def mla(seq, q_lens=None, H=128, P=64, seed=13, q_scale=1.0, causal=True, n_ext=0):
    return wl.build(f"mla-h{H}-p{P}", dtype="bf16", mla=True, seq_lens=seq, q_lens=q_lens,
                    num_q_heads=H, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P,
                    scale=wl.MLA_SCALE, seed=seed, value_scale=0.1, q_scale=q_scale, causal=causal,
                    n_ext=n_ext, ext_lse_center=5.0)


RAGGED = [1, 31, 32, 33, 63, 64, 65, 200, 1000, 2049]


@pytest.mark.parametrize("sharp", [False, True])
@pytest.mark.parametrize("P", [64, 32, 16])
def test_mla_ragged(sharp, P):
    w = mla(RAGGED, P=P, q_scale=wl.SHARP_MLA if sharp else 1.0, seed=P + sharp)
    rng = np.random.default_rng(P)
    counts = [int(rng.integers(1, (L + 63) // 64 + 1)) for L in RAGGED]
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), counts))


@pytest.mark.parametrize("H", [16, 64, 96])
def test_mla_fewer_heads(H):
    w = mla([100, 700, 64], H=H, seed=H, q_scale=wl.SHARP_MLA)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256))


def test_mla_causal_chunk_rows():
    # a chunked-prefill request (40 new tokens over 500 cached) next to decode rows
    w = mla([540, 333, 70], q_lens=[40, 1, 3], seed=3, q_scale=wl.SHARP_MLA)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 2, 2], q_lens=w.q_lens))
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens), check_partials=False)


def test_mla_permuted_equals_identity_bitwise():
    w = mla(RAGGED, seed=5)
    wi = wl.identity_layout(w)
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [1, 1, 1, 1, 1, 1, 2, 3, 5, 9])
    for x, y in zip(run_path(w, plan), run_path(wi, plan)):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))


def test_mla_coverage_probe():
    seq = [1000, 2049, 65, 4000]
    w = mla(seq, seed=9)
    w.q[...] = 0
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [3, 7, 2, 13])
    ranges = plan.ranges()
    xs_all = []
    for b, L in enumerate(seq):
        xs = set()
        for a0, e0 in ranges[b]:
            for x in (a0 - 1, a0, a0 + 1, e0 - 1, e0, e0 + 1):
                if 0 <= x <= L:
                    xs.add(x)
        xs = sorted(xs)[:512]
        xs = np.array(xs + [L] * (512 - len(xs)))
        xs_all.append(xs)
        vals = (np.arange(L)[:, None] >= xs[None, :]).astype(np.float32)[:, None, :]
        wl.set_logical_values(w, b, wl.f32_to_bf16_bits(np.ascontiguousarray(vals)))
    o_part, lse_part, _, _ = run_path(w, plan)
    e = plan.export()
    for b, L in enumerate(seq):
        off = int(e["state_row_offset"][b])
        for r, (a0, e0) in enumerate(ranges[b]):
            rows = slice(off + r * 128, off + (r + 1) * 128)
            cnt = e0 - a0
            assert np.all(np.rint(np.exp(lse_part[rows])) == cnt)
            want = np.maximum(0, e0 - np.maximum(a0, xs_all[b]))
            assert np.array_equal(np.rint(cnt * o_part[rows]), np.broadcast_to(want, (128, 512)))


def test_mla_external_states():
    w = mla([300, 1000], seed=4, n_ext=16)
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, n_ext=16))


def test_mla_external_states_empty_nan():
    # empty external states (LSE -inf) carrying NaN vectors are not read by the
    # many-state merge; a 3-token request makes the row runs ragged
    w = mla([300, 1000], q_lens=[1, 3], seed=9, n_ext=16)
    mask = np.random.default_rng(5).random(w.lse_ext.shape) < 0.25
    w.lse_ext[mask] = -np.inf
    w.o_ext[mask] = np.nan
    d = DeviceInputs(w)
    w.o_ext[mask] = 0.0
    check_all(w, skv.plan_splits(w.seq_lens, spec_of(w), 256, q_lens=w.q_lens, n_ext=16), d)


@pytest.mark.parametrize("num_cu", [256, 4])
def test_mla_merge_up_to_128_states(num_cu):
    # 512-wide merge with 64 external states and a request in 40 splits (104
    # states per row), single-row units (256 CUs) and multi-row units (4)
    w = mla([2600, 300], q_lens=[1, 12], seed=15, n_ext=64)
    mask = np.random.default_rng(9).random(w.lse_ext.shape) < 0.1
    w.lse_ext[mask] = -np.inf
    w.o_ext[mask] = np.nan
    d = DeviceInputs(w)
    w.o_ext[mask] = 0.0
    plan = skv.plan_from_counts(w.seq_lens, spec_of(w), [40, 3], num_cu, q_lens=w.q_lens, n_ext=64)
    if num_cu == 4:
        assert plan.info().reduction_run >= 8
    check_all(w, plan, d)


def test_mla_deterministic():
    w = mla(RAGGED, seed=21)
    plan = skv.plan_splits(w.seq_lens, spec_of(w), 256)
    d = DeviceInputs(w)
    for x, y in zip(run_path(w, plan, d), run_path(w, plan, d)):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))
    assert plan.read_error_flag() == 0


def _scale_rope(w, b, tokens, c):
    """Multiply the 64 rope columns (key only, not the value) of the given
    tokens of request b."""
    for j in tokens:
        pid, slot = wl.physical_slot(w, b, j)
        rope = (w.k_pages[pid, slot, 512:].astype(np.uint32) << 16).view(np.float32)
        w.k_pages[pid, slot, 512:] = wl.f32_to_bf16_bits(rope * np.float32(c))


@pytest.mark.parametrize("P", [64, 16])
def test_mla_rising_scores(P):
    # a few late tokens with scaled-up rope keys: the maximum score of some
    # heads rises by more than 64 (log2 units) above that of the first tile of
    # their split, which makes the MLA kernel run the split a second time
    w = mla([3000, 1500, 97], P=P, seed=31, q_scale=wl.SHARP_MLA)
    _scale_rope(w, 0, [400, 401], 8.0)
    _scale_rope(w, 0, [1500], 30.0)
    _scale_rope(w, 0, [2900], 90.0)
    _scale_rope(w, 1, [1400], 60.0)
    _scale_rope(w, 2, [96], 60.0)
    check_all(w, skv.plan_from_counts(w.seq_lens, spec_of(w), [2, 1, 1]))
