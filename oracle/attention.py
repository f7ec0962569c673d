"""Plain float64 attention, partial attention states and their LSE merge.

Test infrastructure only (see the package docstring).

Definitions followed
--------------------
* Partial attention state (LiquidCP, section 2.1 "Preliminaries"): for a KV
  subset S_r, the locally normalised output o^(r) together with the log-sum-exp
  of the scores over S_r.
* Composition (LiquidCP, section 3, Equation 1): for a partition {S_r} of the
  valid KV positions of a query, o = sum_r exp(lse_r) o^(r) / sum_r exp(lse_r).
  The Helix deep dive (Flash-Decoding recombination in the attention step)
  describes the same merge as rescaling each partial by exp(lse_r - lse_global)
  and summing, with lse_global the log-sum-exp of the partial LSEs.
* Scores are softmax_scale * <q, k>, natural-log LSE over exactly these scores
  (the Helix step 2 "log of sum of exp of attention scores").
* Causal rows (chunked prefill appended to a cached history): query token i of a
  request with n query tokens and L KV tokens sees positions 0 .. L - n + i
  (the chunk's own KV is the last n positions). Decode (n = 1) sees all L.

Every input is upcast exactly from its stored dtype to float64 before use.

FP8 KV cache (SPLASH appendix C.1 serves its MLA backend from an FP8 E4M3 KV
cache): keys and values are stored as OCP 8-bit floating-point E4M3 codes with
one float32 scale per (page, KV head) for keys and one for values; the value
a code stands for is decoded from the format's definition (``e4m3_value``) and
multiplied by its block's scale, exactly, in float64.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------------
# Storage decoding and page-table gather
# ---------------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast: bf16 bit patterns (uint16) or float32 values to float64.
    An fp8-KV workload's queries are bf16."""
    if dtype in ("bf16", "fp8"):
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """The number an OCP E4M3 code stands for (OCP 8-bit floating point
    specification, E4M3 format): bit 7 is the sign, bits 6-3 the exponent with
    bias 7, bits 2-0 the mantissa. Exponent field 0 encodes subnormals
    (mantissa / 8) * 2^-6; exponent 1..15 encodes (1 + mantissa / 8) * 2^(e - 7),
    except exponent 15 with mantissa 7, which is NaN. There are no infinities:
    the largest finite magnitude is 1.75 * 2^8 = 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


_E4M3 = np.array([e4m3_value(c) for c in range(256)], np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3 codes (uint8) to float64 values."""
    return _E4M3[np.asarray(codes, np.uint8)]


def gather_kv(w, b: int, upto: int | None = None):
    """Logical K [L][H_kv][D] and V [L][H_kv][D_v] of request b, in float64.

    Token j lives in physical page page_table[b][j // P] at slot j % P. GQA keys
    are stored [page][kv_head][D/X][P][X], values [page][kv_head][D_v][P]; MLA
    rows are [page][P][576] and the value is the first D_v entries of the row.
    Only the first ``upto`` tokens (default: all L_b) are gathered.
    """
    P = w.page_size
    L = int(w.seq_lens[b]) if upto is None else int(upto)
    npg = (L + P - 1) // P
    pids = w.page_table[b, :npg].astype(np.int64)
    if w.mla:
        rows = w.k_pages[pids]                              # [npg][P][576]
        if w.dtype == "fp8":
            # every row of a page takes the page's scale
            rows = e4m3_to_f64(rows) * w.k_scale[pids].astype(np.float64)[:, :, None]
        else:
            rows = to_f64(rows, w.dtype)
        rows = rows.reshape(npg * P, 1, w.head_dim_qk)[:L]
        return rows, rows[:, :, : w.head_dim_v]
    k = w.k_pages[pids]                                     # [npg][H][D/X][P][X]
    k = np.transpose(k, (0, 3, 1, 2, 4)).reshape(npg * P, w.num_kv_heads, w.head_dim_qk)
    v = w.v_pages[pids]                                     # [npg][H][D_v][P]
    v = np.transpose(v, (0, 3, 1, 2)).reshape(npg * P, w.num_kv_heads, w.head_dim_v)
    if w.dtype == "fp8":
        # every token of a page takes its page's scale for its KV head
        ks = np.repeat(w.k_scale[pids].astype(np.float64), P, axis=0)   # [npg * P][H]
        vs = np.repeat(w.v_scale[pids].astype(np.float64), P, axis=0)
        return (e4m3_to_f64(k[:L]) * ks[:L, :, None], e4m3_to_f64(v[:L]) * vs[:L, :, None])
    return to_f64(k[:L], w.dtype), to_f64(v[:L], w.dtype)


def q_offsets(w) -> np.ndarray:
    """First query-token index of each request (requests concatenated in batch order)."""
    off = np.zeros(w.batch + 1, np.int64)
    off[1:] = np.cumsum(w.q_lens)
    return off


def visible_end(w, b: int, i: int) -> int:
    """Number of KV positions visible to query token i of request b."""
    L, n = int(w.seq_lens[b]), int(w.q_lens[b])
    return L - n + i + 1 if w.causal else L


# ---------------------------------------------------------------------------------
# Softmax attention over one KV subset
# ---------------------------------------------------------------------------------

def softmax_state(S: np.ndarray, V: np.ndarray):
    """(O, LSE) for each row of scores S [r][m] over values V [m][D_v].

    Row-wise: LSE = log sum_j exp(s_j) (computed as max + log sum exp(s - max));
    O = sum_j exp(s_j - LSE) V_j. An empty subset (m = 0) gives O = 0 and
    LSE = -inf, which contributes nothing to a merge.
    """
    r = S.shape[0]
    if S.shape[1] == 0:
        return np.zeros((r, V.shape[-1])), np.full(r, NEG_INF)
    mx = np.max(S, axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.sum(np.exp(S - mx), axis=1))
    p = np.exp(S - lse[:, None])
    return p @ V, lse


def attention_rows(w, b: int, token_ids, lo: int = 0, hi: int | None = None,
                   K=None, V=None):
    """Attention of the listed query tokens (all heads) of request b over KV
    positions [lo, hi) intersected with each token's visible range.

    Returns O [len(token_ids)][H_q][D_v] and LSE [len(token_ids)][H_q].
    KV head of query head h is h // G (contiguous query-head groups; Helix
    assigns each GPU a contiguous query-head slice with its own KV heads).
    """
    H_q, G, Dv = w.num_q_heads, w.group, w.head_dim_v
    if K is None:
        K, V = gather_kv(w, b)
    L = int(w.seq_lens[b])
    hi = L if hi is None else hi
    qoff = int(q_offsets(w)[b])
    out_o = np.zeros((len(token_ids), H_q, Dv))
    out_l = np.full((len(token_ids), H_q), NEG_INF)
    for t, i in enumerate(token_ids):
        e = min(hi, visible_end(w, b, i))
        if e <= lo:
            continue
        q = to_f64(w.q[qoff + i], w.dtype)                   # [H_q][D]
        for g in range(w.num_kv_heads):
            Kg, Vg = K[lo:e, g, :], V[lo:e, g, :]
            S = w.scale * (q[g * G:(g + 1) * G] @ Kg.T)      # [G][m]
            o, l = softmax_state(S, Vg)
            out_o[t, g * G:(g + 1) * G] = o
            out_l[t, g * G:(g + 1) * G] = l
    return out_o, out_l


def full_attention(w, requests=None, token_ids=None):
    """Exact attention for every row of the listed requests (default: all).

    Returns a dict b -> (O [n_b][H_q][D_v], LSE [n_b][H_q]); ``token_ids`` maps
    b to a subset of query tokens when only some rows are wanted.
    """
    out = {}
    for b in (range(w.batch) if requests is None else requests):
        ids = list(range(int(w.q_lens[b]))) if token_ids is None else list(token_ids[b])
        out[b] = attention_rows(w, b, ids)
    return out


def partial_states(w, b: int, splits, token_ids=None, K=None, V=None):
    """Partial states of request b for the split ranges ``splits`` = [(lo, hi), ...].

    Returns O [s][n][H_q][D_v] and LSE [s][n][H_q] (n = listed query tokens).
    """
    ids = list(range(int(w.q_lens[b]))) if token_ids is None else list(token_ids)
    if K is None:
        K, V = gather_kv(w, b)
    os_, ls_ = [], []
    for lo, hi in splits:
        o, l = attention_rows(w, b, ids, lo, hi, K=K, V=V)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


# ---------------------------------------------------------------------------------
# Merge (composition of partial states)
# ---------------------------------------------------------------------------------

def merge(o_states: np.ndarray, lse_states: np.ndarray):
    """Merge partial states along axis 0.

    o_states [s][...][D_v], lse_states [s][...]. With M = max_r lse_r and
    w_r = exp(lse_r - M): O = sum_r w_r o_r / sum_r w_r and LSE = M + log sum_r w_r.
    Rows whose states are all empty (every lse = -inf) give O = 0, LSE = -inf.
    """
    o_states = np.asarray(o_states, np.float64)
    lse_states = np.asarray(lse_states, np.float64)
    M = np.max(lse_states, axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    wts = np.exp(lse_states - Ms[None])                  # exp(-inf) = 0 for empty states
    Z = np.sum(wts, axis=0)
    Zs = np.where(empty, 1.0, Z)
    o = np.sum(wts[..., None] * o_states, axis=0) / Zs[..., None]
    lse = np.where(empty, NEG_INF, Ms + np.log(Zs))
    o = np.where(empty[..., None], 0.0, o)
    return o, lse
