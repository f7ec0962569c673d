"""Pins for the float64 attention oracle (CPU only).

Every check here compares the oracle with something other than itself:
pure-Python brute force with its own index arithmetic, closed forms, an
independent library routine (torch's CPU scaled_dot_product_attention in
float64), and the composition identity of partial states (LiquidCP section 3,
Equation 1; the Helix deep dive's rescale-and-sum recombination). The last
group plants plausible mistakes in the oracle and checks that a pin fails.
"""
import math
import struct

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as A


# ----------------------------------------------------------------------------------
# independent brute force (pure Python, math.fsum, explicit storage indexing)
# ----------------------------------------------------------------------------------

def _val(w, x) -> float:
    if w.dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    return float(x)


def _key(w, b, j, g, d):
    pid = int(w.page_table[b][j // w.page_size])
    slot = j % w.page_size
    if w.mla:
        return _val(w, w.k_pages[pid][slot][d])
    return _val(w, w.k_pages[pid][g][d // w.x][slot][d % w.x])


def _value(w, b, j, g, d):
    pid = int(w.page_table[b][j // w.page_size])
    slot = j % w.page_size
    if w.mla:
        return _val(w, w.k_pages[pid][slot][d])
    return _val(w, w.v_pages[pid][g][d][slot])


def _query(w, b, i, h, d):
    row = sum(int(x) for x in w.q_lens[:b]) + i
    return _val(w, w.q[row][h][d])


def brute(w, b, i, h, lo=0, hi=None):
    L, n = int(w.seq_lens[b]), int(w.q_lens[b])
    vis = L - n + i + 1 if w.causal else L
    hi = L if hi is None else hi
    e = min(hi, vis)
    g = h // (w.num_q_heads // w.num_kv_heads)
    D, Dv = w.head_dim_qk, w.head_dim_v
    scores = []
    for j in range(lo, e):
        scores.append(w.scale * math.fsum(_query(w, b, i, h, d) * _key(w, b, j, g, d)
                                          for d in range(D)))
    if not scores:
        return [0.0] * Dv, -math.inf
    m = max(scores)
    lse = m + math.log(math.fsum(math.exp(s - m) for s in scores))
    o = [math.fsum(math.exp(s - lse) * _value(w, b, lo + t, g, d) for t, s in enumerate(scores))
         for d in range(Dv)]
    return o, lse


def tiny(dtype="f32", mla=False, seq_lens=(5, 8, 1), q_lens=None, H_q=4, H_kv=2, D=None,
         Dv=None, P=4, seed=7, causal=True, q_scale=1.0):
    if D is None:
        D = 12 if mla else (8 if dtype == "bf16" else 4)
    if Dv is None:
        Dv = 8 if mla else D
    return wl.build("tiny", dtype=dtype, mla=mla, seq_lens=list(seq_lens), q_lens=q_lens,
                    num_q_heads=H_q, num_kv_heads=1 if mla else H_kv, head_dim_qk=D,
                    head_dim_v=Dv, page_size=P, scale=0.7, seed=seed, causal=causal,
                    q_scale=q_scale)


TINY_CASES = [
    dict(dtype="f32"),
    dict(dtype="bf16"),
    dict(dtype="f32", mla=True, H_q=3),
    dict(dtype="bf16", mla=True, H_q=2),
    dict(dtype="f32", seq_lens=(7, 4), q_lens=(3, 4)),          # causal chunk rows
    dict(dtype="bf16", seq_lens=(6,), q_lens=(2,), causal=False),
    dict(dtype="f32", H_q=6, H_kv=3, P=2, seq_lens=(3, 2, 8)),
]


def pin_bruteforce(w, att=A) -> float:
    """Max abs difference between the oracle and brute force over every row."""
    err = 0.0
    res = att.full_attention(w)
    for b in range(w.batch):
        o, l = res[b]
        for i in range(int(w.q_lens[b])):
            for h in range(w.num_q_heads):
                bo, bl = brute(w, b, i, h)
                err = max(err, abs(l[i, h] - bl), float(np.max(np.abs(o[i, h] - bo))))
    return err


@pytest.mark.parametrize("case", TINY_CASES)
def test_bruteforce(case):
    w = tiny(**case)
    assert pin_bruteforce(w) <= 1e-12


@pytest.mark.parametrize("case", TINY_CASES[:4])
def test_bruteforce_partial(case):
    w = tiny(**case)
    b = int(np.argmax(w.seq_lens))
    L = int(w.seq_lens[b])
    splits = [(0, 1), (1, 1), (1, L - 2), (L - 2, L)]    # includes an empty split
    o, l = A.partial_states(w, b, splits)
    for r, (lo, hi) in enumerate(splits):
        for h in range(w.num_q_heads):
            bo, bl = brute(w, b, 0, h, lo, hi)
            if math.isinf(bl):
                assert np.isneginf(l[r, 0, h]) and np.all(o[r, 0, h] == 0)
            else:
                assert abs(l[r, 0, h] - bl) <= 1e-12
                assert np.max(np.abs(o[r, 0, h] - bo)) <= 1e-12


# ----------------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------------

def _scores(w, b, i, h):
    L = int(w.seq_lens[b])
    g = h // w.group
    return [w.scale * sum(_query(w, b, i, h, d) * _key(w, b, j, g, d)
                          for d in range(w.head_dim_qk)) for j in range(L)]


def test_single_token():
    w = tiny(seq_lens=(1, 1), H_q=2, H_kv=1)
    res = A.full_attention(w)
    for b in range(2):
        for h in range(2):
            s = _scores(w, b, 0, h)[0]
            v = [_value(w, b, 0, 0, d) for d in range(w.head_dim_v)]
            assert abs(res[b][1][0, h] - s) <= 1e-12
            assert np.max(np.abs(res[b][0][0, h] - v)) <= 1e-15


def test_two_tokens_sigmoid():
    w = tiny(seq_lens=(2,), H_q=3, H_kv=1, q_scale=2.0)
    o, l = A.full_attention(w)[0]
    for h in range(3):
        s0, s1 = _scores(w, 0, 0, h)
        sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        v0 = np.array([_value(w, 0, 0, 0, d) for d in range(w.head_dim_v)])
        v1 = np.array([_value(w, 0, 1, 0, d) for d in range(w.head_dim_v)])
        assert np.max(np.abs(o[0, h] - (sig * v0 + (1 - sig) * v1))) <= 1e-14
        assert abs(l[0, h] - np.logaddexp(s0, s1)) <= 1e-14


def test_zero_query_is_mean():
    w = tiny(seq_lens=(9, 3), H_q=2, H_kv=1, causal=False)
    w.q[...] = 0
    res = A.full_attention(w)
    for b in range(2):
        L = int(w.seq_lens[b])
        vm = np.array([[_value(w, b, j, 0, d) for d in range(w.head_dim_v)] for j in range(L)])
        for h in range(2):
            assert abs(res[b][1][0, h] - math.log(L)) <= 1e-14
            assert np.max(np.abs(res[b][0][0, h] - vm.mean(axis=0))) <= 1e-14


def test_constant_values():
    w = tiny(seq_lens=(11,), H_q=2, H_kv=1, P=4)
    const = np.linspace(-1.0, 1.0, w.head_dim_v).astype(np.float32)
    wl.set_logical_values(w, 0, np.broadcast_to(const, (11, 1, w.head_dim_v)))
    o, _ = A.full_attention(w)[0]
    assert np.max(np.abs(o[0] - const[None].astype(np.float64))) <= 1e-14


# ----------------------------------------------------------------------------------
# independent library routine: torch CPU SDPA in float64
# ----------------------------------------------------------------------------------

def _dense(w, b):
    L = int(w.seq_lens[b])
    K = np.array([[[_key(w, b, j, g, d) for d in range(w.head_dim_qk)]
                   for g in range(w.num_kv_heads)] for j in range(L)])
    V = np.array([[[_value(w, b, j, g, d) for d in range(w.head_dim_v)]
                   for g in range(w.num_kv_heads)] for j in range(L)])
    return K, V


@pytest.mark.parametrize("dtype,mla", [("f32", False), ("bf16", False), ("bf16", True)])
def test_torch_sdpa_decode(dtype, mla):
    w = tiny(dtype=dtype, mla=mla, seq_lens=(13, 6), H_q=4, H_kv=2,
             D=16 if not mla else 12, Dv=16 if not mla else 8, P=4)
    res = A.full_attention(w)
    for b in range(w.batch):
        K, V = _dense(w, b)
        q = np.array([[_query(w, b, 0, h, d) for d in range(w.head_dim_qk)]
                      for h in range(w.num_q_heads)])
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(w.group, 0)[None]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(w.group, 0)[None]
        qt = torch.from_numpy(q)[None, :, None, :]
        out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=w.scale)
        assert np.max(np.abs(res[b][0][0] - out[0, :, 0, :].numpy())) <= 1e-13


def test_torch_sdpa_causal_square():
    # With n = L the bottom-right causal rule is the ordinary causal mask.
    w = tiny(seq_lens=(6,), q_lens=(6,), H_q=2, H_kv=1, D=8, P=4)
    o, _ = A.full_attention(w)[0]
    K, V = _dense(w, 0)
    q = np.array([[[_query(w, 0, i, h, d) for d in range(8)] for i in range(6)]
                  for h in range(2)])
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K).permute(1, 0, 2).repeat(2, 1, 1)[None],
        torch.from_numpy(V).permute(1, 0, 2).repeat(2, 1, 1)[None], is_causal=True, scale=w.scale)
    assert np.max(np.abs(o - out[0].permute(1, 0, 2).numpy())) <= 1e-13


# ----------------------------------------------------------------------------------
# composition of partial states (LiquidCP Equation 1) and merge identities
# ----------------------------------------------------------------------------------

def _random_splits(rng, L):
    cuts = sorted(rng.integers(0, L + 1, size=rng.integers(1, 6)).tolist())
    bounds = [0] + cuts + [L]
    return [(bounds[k], bounds[k + 1]) for k in range(len(bounds) - 1)]


@pytest.mark.parametrize("seed", range(6))
def test_split_merge_equals_full(seed):
    rng = np.random.default_rng(seed)
    mla = seed % 3 == 2
    w = tiny(dtype="bf16" if seed % 2 else "f32", mla=mla, seq_lens=(37, 20),
             q_lens=(3, 1), H_q=4, H_kv=2, P=4 + 4 * (seed % 2), seed=seed, q_scale=3.0)
    full = A.full_attention(w)
    for b in range(w.batch):
        splits = _random_splits(rng, int(w.seq_lens[b]))
        o, l = A.partial_states(w, b, splits)
        order = rng.permutation(len(splits))
        mo, ml = A.merge(o[order], l[order])
        assert np.max(np.abs(mo - full[b][0])) <= 1e-12
        assert np.max(np.abs(ml - full[b][1])) <= 1e-12


def test_merge_identities():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((3, 5, 7))
    l = rng.standard_normal((3, 5))
    base_o, base_l = A.merge(o, l)
    # an empty state (O = 0, LSE = -inf) is the identity
    o2 = np.concatenate([o, np.zeros((1, 5, 7))])
    l2 = np.concatenate([l, np.full((1, 5), -np.inf)])
    mo, ml = A.merge(o2, l2)
    assert np.max(np.abs(mo - base_o)) <= 1e-15 and np.max(np.abs(ml - base_l)) <= 1e-15
    # two states with equal LSE: their average, and LSE + ln 2
    mo, ml = A.merge(o[:2], np.stack([l[0], l[0]]))
    assert np.max(np.abs(mo - 0.5 * (o[0] + o[1]))) <= 1e-15
    assert np.max(np.abs(ml - (l[0] + math.log(2.0)))) <= 1e-14
    # all-empty rows give (0, -inf)
    mo, ml = A.merge(np.ones((2, 1, 3)), np.full((2, 1), -np.inf))
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # explicit weights for one row: exp-weighted average of the outputs
    wts = np.exp(l[:, 0]) / np.exp(l[:, 0]).sum()
    assert np.max(np.abs(base_o[0] - (wts[:, None] * o[:, 0]).sum(0))) <= 1e-14
    assert abs(base_l[0] - math.log(np.exp(l[:, 0]).sum())) <= 1e-14


# ----------------------------------------------------------------------------------
# page-table indexing
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,mla", [("f32", False), ("bf16", False), ("bf16", True)])
def test_gather_permuted_equals_identity(dtype, mla):
    w = tiny(dtype=dtype, mla=mla, seq_lens=(23, 5, 16), P=4)
    wi = wl.identity_layout(w)
    assert not np.array_equal(w.page_table, wi.page_table)
    for b in range(w.batch):
        k1, v1 = A.gather_kv(w, b)
        k2, v2 = A.gather_kv(wi, b)
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
        K, V = _dense(w, b)
        assert np.array_equal(k1, K) and np.array_equal(v1, V)
        assert not np.isnan(k1).any() and not np.isnan(v1).any()


def test_unused_slots_poisoned():
    # the generator poisons every slot past L_b; the oracle must never read one
    w = tiny(seq_lens=(5, 9), P=4)
    pid = int(w.page_table[0][1])
    assert np.isnan(w.k_pages[pid][:, :, 1:, :]).all()
    assert not np.isnan(w.k_pages[pid][:, :, :1, :]).any()
    res = A.full_attention(w)
    assert all(np.isfinite(res[b][0]).all() for b in res)


# ----------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    w = tiny(dtype="f32", seq_lens=(7, 4), q_lens=(3, 2), H_q=4, H_kv=2, P=4)
    assert pin_bruteforce(w) <= 1e-12

    def caught(patch_target, patch):
        with monkeypatch.context() as m:
            m.setattr(A, patch_target, patch)
            return pin_bruteforce(w) > 1e-6

    orig_vis, orig_soft, orig_gather = A.visible_end, A.softmax_state, A.gather_kv
    # off-by-one causal boundary
    assert caught("visible_end", lambda w_, b, i: orig_vis(w_, b, i) - 1)
    # log-sum-exp without the max shift added back
    def lse_drop_max(S, V):
        o, l = orig_soft(S, V)
        return o, l - np.max(S, axis=1)
    assert caught("softmax_state", lse_drop_max)
    # keys read in reversed token order (wrong page/slot indexing)
    def bad_gather(w_, b, upto=None):
        k, v = orig_gather(w_, b, upto)
        return k[::-1].copy(), v
    assert caught("gather_kv", bad_gather)
    # wrong head-to-KV-head mapping (interleaved instead of contiguous groups)
    def interleaved(w_, b, token_ids, lo=0, hi=None, K=None, V=None):
        K, V = orig_gather(w_, b)
        return orig_attention(w_, b, token_ids, lo, hi, K=K[:, ::-1].copy(), V=V[:, ::-1].copy())
    orig_attention = A.attention_rows
    assert caught("attention_rows", interleaved)


def test_planted_merge_mistake_is_caught(monkeypatch):
    w = tiny(dtype="f32", seq_lens=(29,), H_q=2, H_kv=1, P=4, q_scale=3.0)
    full_o, full_l = A.full_attention(w)[0]
    splits = [(0, 5), (5, 17), (17, 29)]
    o, l = A.partial_states(w, 0, splits)
    mo, _ = A.merge(o, l)
    assert np.max(np.abs(mo - full_o)) <= 1e-12
    orig_exp = np.exp

    def flipped(x, *a, **k):            # exp(M - lse) instead of exp(lse - M)
        return orig_exp(-x, *a, **k)
    with monkeypatch.context() as m:
        m.setattr(A.np, "exp", flipped)
        bad_o, _ = A.merge(o, l)
    assert np.max(np.abs(bad_o - full_o)) > 1e-6
