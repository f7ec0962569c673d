"""Pins of the oracle's FP8 (OCP E4M3) KV decoding, on the CPU.

The decoder is written from the format's definition (oracle.attention.e4m3_value).
It is pinned to values the definition fixes (zero, the smallest subnormal, the
smallest normal, one, the largest finite value, the NaN codes), to its
structure (monotone over the positive codes, constant spacing inside each
binade, sign symmetry), to an independent implementation (PyTorch's
float8_e4m3fn conversion, all 256 codes), and each planted mistake below fails
at least one pin. The paged gather of an FP8 workload is checked by brute force
against a per-element loop, and attention over it equals attention over an fp32
workload that stores the decoded values; the same for FP8 MLA latent rows, whose
one scale per page covers both the keys and the values (the rows' first 512
codes)."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as A


def _pins_hold(dec) -> bool:
    """Every value-level pin for a candidate decoder dec(code) -> float."""
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    if any(dec(c) != v for c, v in fixed.items()):
        return False
    if not (math.isnan(dec(0x7F)) and math.isnan(dec(0xFF))):
        return False
    if not (dec(0x80) == 0.0 and math.copysign(1.0, dec(0x80)) < 0):
        return False
    pos = [dec(c) for c in range(0x7F)]
    if any(b <= a for a, b in zip(pos, pos[1:])):
        return False
    for c in range(0x7F):   # sign symmetry
        if dec(c | 0x80) != -dec(c):
            return False
    # constant spacing inside each binade: 2^(e - 10) for e >= 1, 2^-9 below
    for e in range(16):
        codes = [c for c in range(0x7F) if (c >> 3) == e]
        vals = [dec(c) for c in codes]
        step = 2.0 ** (max(e, 1) - 10)
        if any(b - a != step for a, b in zip(vals, vals[1:])):
            return False
    return True


def test_decoder_pins():
    assert _pins_hold(A.e4m3_value)


def test_decoder_matches_pytorch_float8_e4m3fn_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = A.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def _planted():
    def bias8(c):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            return math.nan
        return s * (math.ldexp(m / 8.0, -7) if e == 0 else math.ldexp(1 + m / 8.0, e - 8))

    def no_subnormals(c):
        return 0.0 if (c >> 3) & 15 == 0 else A.e4m3_value(c)

    def subnormal_exp_minus7(c):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        return s * math.ldexp(m / 8.0, -7) if e == 0 else A.e4m3_value(c)

    def e5m2_style_nan(c):   # whole top binade taken as non-finite, as in IEEE-like formats
        return math.nan if (c >> 3) & 15 == 15 else A.e4m3_value(c)

    def mantissa_over_16(c):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            return math.nan
        return s * (math.ldexp(m / 16.0, -6) if e == 0 else math.ldexp(1 + m / 16.0, e - 7))

    def sign_dropped(c):
        return abs(A.e4m3_value(c))

    return [bias8, no_subnormals, subnormal_exp_minus7, e5m2_style_nan, mantissa_over_16, sign_dropped]


@pytest.mark.parametrize("dec", _planted(), ids=lambda f: f.__name__)
def test_planted_decoder_mistakes_fail_a_pin(dec):
    assert not _pins_hold(dec)


def _fp8_case(seed=3, P=16, D=64):
    return wl.build("fp8-small", dtype="fp8", mla=False, seq_lens=[37, 16, 90], q_lens=[1, 2, 1],
                    num_q_heads=16, num_kv_heads=2, head_dim_qk=D, head_dim_v=D, page_size=P,
                    scale=1.0 / math.sqrt(D), seed=seed)


def test_generator_codes_and_scales():
    w = _fp8_case()
    assert w.k_pages.dtype == np.uint8 and w.k_pages.shape[2:] == (64 // 16, 16, 16)
    assert w.v_pages.dtype == np.uint8 and w.k_scale.shape == (w.num_pages, 2)
    used = w.logical_to_physical
    assert np.all(w.k_scale[used] > 0) and np.all(np.isfinite(w.v_scale[used]))
    # each used block's largest magnitude maps to the format's largest finite value
    vals = A.e4m3_to_f64(w.k_pages[used])
    assert np.nanmax(np.abs(vals)) == 448.0


def test_gather_fp8_brute_force():
    w = _fp8_case()
    P, D = w.page_size, w.head_dim_qk
    for b in range(w.batch):
        K, V = A.gather_kv(w, b)
        L = int(w.seq_lens[b])
        assert K.shape == (L, 2, D)
        for j in range(L):
            pid = int(w.page_table[b, j // P])
            s = j % P
            for h in range(2):
                for d in (0, 5, 17, D - 1):
                    kc = int(w.k_pages[pid, h, d // 16, s, d % 16])
                    vc = int(w.v_pages[pid, h, d, s])
                    assert K[j, h, d] == A.e4m3_value(kc) * float(w.k_scale[pid, h])
                    assert V[j, h, d] == A.e4m3_value(vc) * float(w.v_scale[pid, h])


def test_fp8_attention_equals_fp32_on_decoded_values():
    # an fp32 workload that stores the fp8 workload's decoded values, each
    # code's value times its float32 scale rounded to float32 (the product has
    # up to 4 + 24 significant bits): the two agree to that rounding
    w = _fp8_case(seed=9)
    N, H, D, P = w.num_pages, w.num_kv_heads, w.head_dim_qk, w.page_size
    kd = A.e4m3_to_f64(w.k_pages) * w.k_scale.astype(np.float64)[:, :, None, None, None]
    vd = A.e4m3_to_f64(w.v_pages) * w.v_scale.astype(np.float64)[:, :, None, None]
    k32 = kd.reshape(N, H, D // 16, P, 16).transpose(0, 1, 3, 2, 4).reshape(N, H, P, D)
    k32 = k32.reshape(N, H, P, D // 4, 4).transpose(0, 1, 3, 2, 4).astype(np.float32)
    wf = wl.Workload(**{**w.__dict__})
    wf.dtype = "f32"
    wf.q = A.to_f64(w.q, "fp8").astype(np.float32)          # bf16 -> f32 is exact
    wf.k_pages, wf.v_pages = k32, vd.astype(np.float32)
    wf.k_scale = wf.v_scale = None
    for b in range(w.batch):
        ids = list(range(int(w.q_lens[b])))
        o8, l8 = A.attention_rows(w, b, ids)
        of, lf = A.attention_rows(wf, b, ids)
        # the only difference is the float32 rounding of code * scale
        assert np.allclose(o8, of, rtol=1e-6, atol=1e-6) and np.allclose(l8, lf, rtol=1e-6, atol=1e-6)


def _fp8_mla_case(seed=4, P=16, heads=16):
    return wl.build("fp8-mla-small", dtype="fp8", mla=True, seq_lens=[37, 16, 90], q_lens=[1, 2, 1],
                    num_q_heads=heads, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P,
                    scale=1.0 / math.sqrt(192.0), seed=seed, value_scale=0.1)


def test_mla_generator_codes_and_scales():
    w = _fp8_mla_case()
    assert w.k_pages.dtype == np.uint8 and w.k_pages.shape == (w.num_pages, 16, 576)
    assert w.v_pages is None and w.k_scale.shape == (w.num_pages, 1) and w.v_scale is w.k_scale
    used = w.logical_to_physical
    assert np.all(w.k_scale[used] > 0)
    # one scale per page: the largest magnitude of each fully used page maps to
    # 448 (the tail slots of a request's last page are poisoned after scaling)
    P = w.page_size
    full = [int(w.page_table[b, p]) for b in range(w.batch) for p in range(int(w.seq_lens[b]) // P)]
    vals = A.e4m3_to_f64(w.k_pages[full]).reshape(len(full), -1)
    assert len(full) >= 4 and np.all(np.max(np.abs(vals), axis=1) == 448.0)
    spare = np.setdiff1d(np.arange(w.num_pages), used)
    assert np.all(np.isnan(w.k_scale[spare]))


def test_mla_gather_fp8_brute_force():
    # a latent row is its codes' E4M3 values times its page's scale; the value
    # is the row's first 512 entries
    w = _fp8_mla_case()
    P = w.page_size
    for b in range(w.batch):
        K, V = A.gather_kv(w, b)
        L = int(w.seq_lens[b])
        assert K.shape == (L, 1, 576) and V.shape == (L, 1, 512)
        for j in range(L):
            pid = int(w.page_table[b, j // P])
            for d in (0, 7, 300, 511, 512, 575):
                want = A.e4m3_value(int(w.k_pages[pid, j % P, d])) * float(w.k_scale[pid, 0])
                assert K[j, 0, d] == want
                if d < 512:
                    assert V[j, 0, d] == want


def test_mla_fp8_attention_equals_fp32_on_decoded_values():
    # an fp32 MLA workload storing the decoded rows (code value times scale,
    # rounded to float32) agrees with the FP8 one to that rounding
    w = _fp8_mla_case(seed=10)
    kd = A.e4m3_to_f64(w.k_pages) * w.k_scale.astype(np.float64)[:, :, None]
    wf = wl.Workload(**{**w.__dict__})
    wf.dtype = "f32"
    wf.q = A.to_f64(w.q, "fp8").astype(np.float32)
    wf.k_pages = kd.astype(np.float32)
    wf.k_scale = wf.v_scale = None
    for b in range(w.batch):
        ids = list(range(int(w.q_lens[b])))
        o8, l8 = A.attention_rows(w, b, ids)
        of, lf = A.attention_rows(wf, b, ids)
        assert np.allclose(o8, of, rtol=1e-6, atol=1e-7) and np.allclose(l8, lf, rtol=1e-6, atol=1e-6)


def test_mla_fp8_scale_is_per_page():
    # doubling one page's scale doubles exactly the rows of that page
    w = _fp8_mla_case(seed=11)
    b = 2
    K0, _ = A.gather_kv(w, b)
    pid = int(w.page_table[b, 1])
    w.k_scale = w.k_scale.copy()
    w.k_scale[pid, 0] *= 2
    w.v_scale = w.k_scale
    K1, _ = A.gather_kv(w, b)
    P = w.page_size
    assert np.array_equal(K1[P:2 * P], 2 * K0[P:2 * P])
    assert np.array_equal(K1[:P], K0[:P]) and np.array_equal(K1[2 * P:], K0[2 * P:])
