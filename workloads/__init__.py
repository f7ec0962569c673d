"""Seeded synthetic inputs for split-KV decode attention.

This module only draws random numbers and lays them out in the paged-KV storage
formats that the library defines. It contains none of the attention arithmetic:
no dot products, no softmax, no merging. The float64 oracle and the HIP path
both consume exactly the arrays produced here (the oracle through numpy, the HIP
path after a host-to-device copy), which is the only thing the two sides share.

Storage formats (the library's paged KV cache; the pages describe paged KV but
fix no memory layout, so this one is chosen to make every device load a single
coalesced access in the matrix-core operand order):

* GQA keys   ``k_pages[num_pages][H_kv][D / X][P][X]``  with X = 16 bytes / element
  size (X = 8 for bf16, X = 4 for fp32): each 16-byte chunk of X consecutive
  dimensions of one token is contiguous, and the P tokens of a page sit next to
  each other for a fixed chunk.
* GQA values ``v_pages[num_pages][H_kv][D_v][P]``: per page and head, the values
  are stored transposed (dimension-major, tokens contiguous).
* MLA latent ``kv_pages[num_pages][P][576]``: one row per token, the 512-wide
  latent followed by the 64-wide rotary part. The value of a token is the first
  512 entries of its own row (absorbed multi-head latent attention: SPLASH,
  section 2, KV bytes per token L(d_c + d_r)b, and section 3, the owner computes
  rows [N_r, H, d_c + d_r] and returns width d_c).

bf16 arrays are carried as ``numpy.uint16`` bit patterns; fp32 as ``float32``.

FP8 KV (``dtype="fp8"``): queries are bf16; keys and values are OCP E4M3 codes
(``numpy.uint8``) in the GQA layouts above with X = 16, and every (page, KV
head) block has a float32 scale for its keys and one for its values
(``k_scale`` / ``v_scale`` ``[num_pages][H_kv]``): the stored value is
code_value * scale. MLA latent rows in FP8 keep the ``[num_pages][P][576]``
layout with one scale per page (``k_scale [num_pages][1]``; ``v_scale`` is the
same array, the values being the rows' first 512 codes). They are drawn as the float32 normals described below,
divided by their block's max |x| / 448 (so the block's largest value maps to
E4M3's largest finite value) and cast to E4M3 by PyTorch's float8_e4m3fn
conversion (round to nearest even). Unused slots hold the NaN code 0x7F and the
spare pages' scales are NaN.

Random recipe (fixed, so that every consumer sees the same bits): one
``SeedSequence(20260922 + config_id)`` (the base is the residency-sampler seed
printed in SPLASH appendix B.1) spawns independent children for lengths,
request order, page permutation, Q, K, V, external O and external LSE. Large
arrays are drawn in fixed chunks of 2**22 values, each chunk from its own
spawned child, as float32 standard normals, multiplied by the value scale in
float32 and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260922
CHUNK = 1 << 22
BF16_NAN = np.uint16(0x7FC0)

_STREAMS = ("lengths", "order", "pages", "q", "k", "v", "o_ext", "lse_ext")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> 16) & 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def fill_normal(out: np.ndarray, seed: np.random.SeedSequence, scale: float = 1.0,
                offset: float = 0.0) -> None:
    """Fill ``out`` (flat view; uint16 = bf16 bits, or float32) with offset + scale * N(0, 1)."""
    flat = out.reshape(-1)
    n = flat.size
    if n == 0:
        return
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = seed.spawn(nchunks)
    bf16 = flat.dtype == np.uint16

    def work(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        tmp = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            tmp *= np.float32(scale)
        if offset != 0.0:
            tmp += np.float32(offset)
        if bf16:
            flat[lo:hi] = f32_to_bf16_bits(tmp)
        else:
            flat[lo:hi] = tmp

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


@dataclass
class Workload:
    """One batch of decode-attention inputs in the library's storage formats."""
    name: str
    dtype: str                      # "f32", "bf16" or "fp8" (bf16 queries, E4M3 KV)
    mla: bool
    causal: bool
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    seq_lens: np.ndarray            # int32 [B]
    q_lens: np.ndarray              # int32 [B]
    page_table: np.ndarray          # int32 [B][max_pages]
    num_pages: int
    q: np.ndarray                   # [sum q_lens][H_q][D]  (uint16 bits or float32)
    k_pages: np.ndarray             # GQA [N][H_kv][D/X][P][X]; MLA [N][P][576]
    v_pages: np.ndarray | None      # GQA [N][H_kv][D_v][P];   MLA None (aliases k_pages)
    scale: float
    logical_to_physical: np.ndarray  # int32 [num used pages]: physical id of logical page i
    page_offsets: np.ndarray        # int32 [B + 1]: first logical page of each request
    n_ext: int = 0
    o_ext: np.ndarray | None = None    # float32 [n_ext][total_rows][D_v]
    lse_ext: np.ndarray | None = None  # float32 [n_ext][total_rows]
    chunk_tokens: int | None = None    # explicit fixed-chunk split plan, if the config asks for one
    k_scale: np.ndarray | None = None  # fp8: float32 [N][H_kv], key scale per page and KV head
    v_scale: np.ndarray | None = None  # fp8: float32 [N][H_kv], value scale (MLA: k_scale itself)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def total_rows(self) -> int:
        return self.total_q * self.num_q_heads

    @property
    def x(self) -> int:
        return 16 // KV_BYTES[self.dtype]

    def kv_bytes_per_token(self) -> float:
        """KV bytes per token (fp8: plus its share of the per-page scales)."""
        b = KV_BYTES[self.dtype]
        if self.mla:
            return self.head_dim_qk * b + (4 / self.page_size if self.dtype == "fp8" else 0)
        per = self.num_kv_heads * (self.head_dim_qk + self.head_dim_v) * b
        if self.dtype == "fp8":
            per += self.num_kv_heads * 8 / self.page_size
        return per


KV_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
FP8_NAN = np.uint8(0x7F)
FP8_MAX = 448.0


def _poison_value(dtype: str):
    return {"bf16": BF16_NAN, "fp8": FP8_NAN}.get(dtype, np.float32(np.nan))


def _fp8_blocks(x: np.ndarray, out: np.ndarray, scale: np.ndarray, pages_per_pass: int = 4096) -> None:
    """E4M3 codes of x [N][H][...] (float32) into out (uint8, same shape), with
    one scale per [page][head] block: scale = max |x| / 448 (1 for an all-zero
    block), code = E4M3(x / scale) by PyTorch's cast (nearest, ties to even)."""
    import torch
    N = x.shape[0]
    for lo in range(0, N, pages_per_pass):
        hi = min(N, lo + pages_per_pass)
        blk = x[lo:hi]
        amax = np.abs(blk).reshape(hi - lo, blk.shape[1], -1).max(axis=2)
        s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        scale[lo:hi] = s
        shape = (hi - lo, blk.shape[1]) + (1,) * (blk.ndim - 2)
        # |x / scale| <= 448 up to one float32 rounding, which the cast takes to 448
        y = blk / s.reshape(shape)
        out[lo:hi] = torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()


def build(name: str, *, dtype: str, mla: bool, seq_lens, q_lens=None, num_q_heads: int,
          num_kv_heads: int, head_dim_qk: int, head_dim_v: int, page_size: int,
          scale: float, seed: int, value_scale: float = 1.0, q_scale: float = 1.0,
          causal: bool = True, n_ext: int = 0, ext_lse_center: float = 0.0,
          chunk_tokens: int | None = None, spare_pages: int | None = None,
          shuffle: bool = False, lengths_given: bool = True) -> Workload:
    """Draw one workload. ``seq_lens`` are the KV lengths (history plus the query
    tokens' own KV); ``q_lens`` default to one query token per request."""
    ss = np.random.SeedSequence(seed)
    kids = dict(zip(_STREAMS, ss.spawn(len(_STREAMS))))
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = seq_lens.shape[0]
    q_lens = np.ones(B, np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    if shuffle:
        order = np.random.Generator(np.random.PCG64(kids["order"])).permutation(B)
        seq_lens, q_lens = seq_lens[order], q_lens[order]
    assert np.all(seq_lens >= q_lens) and np.all(q_lens >= 1)
    P = page_size
    pages_b = (seq_lens + P - 1) // P
    n_used = int(pages_b.sum())
    n_spare = max(2, n_used // 256) if spare_pages is None else spare_pages
    N = n_used + n_spare
    perm = np.random.Generator(np.random.PCG64(kids["pages"])).permutation(N).astype(np.int32)
    l2p = perm[:n_used]
    spare = perm[n_used:]
    offsets = np.zeros(B + 1, np.int64)
    offsets[1:] = np.cumsum(pages_b)
    max_pages = int(pages_b.max())
    # Entries past a request's last page are never consumed; they point at a
    # poisoned spare page so that any stray use shows up as NaN.
    table = np.full((B, max_pages), spare[0] if n_spare > 0 else 0, np.int32)
    for b in range(B):
        table[b, : pages_b[b]] = l2p[offsets[b]: offsets[b + 1]]

    el = np.uint16 if dtype == "bf16" else np.float32
    H_q, H_kv = num_q_heads, num_kv_heads
    total_q = int(q_lens.sum())
    q = np.empty((total_q, H_q, head_dim_qk), np.uint16 if dtype == "fp8" else el)
    fill_normal(q, kids["q"], scale=value_scale * q_scale)
    k_scale = v_scale = None
    if dtype == "fp8" and mla:
        # one block (and one scale) per page: the page's 576-wide rows, whose
        # first 512 entries are also the values
        assert H_kv == 1
        k32 = np.empty((N, 1, P, head_dim_qk), np.float32)
        fill_normal(k32, kids["k"], scale=value_scale)
        codes = np.empty(k32.shape, np.uint8)
        k_scale = np.empty((N, 1), np.float32)
        _fp8_blocks(k32, codes, k_scale)
        del k32
        k_pages = codes.reshape(N, P, head_dim_qk)
        v_pages = None
        k_scale[spare] = np.nan
        v_scale = k_scale
    elif dtype == "fp8":
        assert head_dim_qk % 16 == 0
        X = 16
        k32 = np.empty((N, H_kv, head_dim_qk // X, P, X), np.float32)
        v32 = np.empty((N, H_kv, head_dim_v, P), np.float32)
        fill_normal(k32, kids["k"], scale=value_scale)
        fill_normal(v32, kids["v"], scale=value_scale)
        k_pages = np.empty(k32.shape, np.uint8)
        v_pages = np.empty(v32.shape, np.uint8)
        k_scale = np.empty((N, H_kv), np.float32)
        v_scale = np.empty((N, H_kv), np.float32)
        _fp8_blocks(k32, k_pages, k_scale)
        _fp8_blocks(v32, v_pages, v_scale)
        del k32, v32
        k_scale[spare] = np.nan
        v_scale[spare] = np.nan
    elif mla:
        assert H_kv == 1
        k_pages = np.empty((N, P, head_dim_qk), el)
        fill_normal(k_pages, kids["k"], scale=value_scale)
        v_pages = None
    else:
        X = 16 // np.dtype(el).itemsize
        assert head_dim_qk % X == 0
        k_pages = np.empty((N, H_kv, head_dim_qk // X, P, X), el)
        v_pages = np.empty((N, H_kv, head_dim_v, P), el)
        fill_normal(k_pages, kids["k"], scale=value_scale)
        fill_normal(v_pages, kids["v"], scale=value_scale)
    poison = _poison_value(dtype)
    # Poison every slot that holds no token: spare pages entirely, and the tail
    # slots of each request's last page.
    for pid in spare:
        k_pages[pid] = poison
        if v_pages is not None:
            v_pages[pid] = poison
    for b in range(B):
        used = int(seq_lens[b] - (pages_b[b] - 1) * P)
        if used < P:
            pid = table[b, pages_b[b] - 1]
            if mla:
                k_pages[pid, used:, :] = poison
            else:
                k_pages[pid, :, :, used:, :] = poison
                v_pages[pid, :, :, used:] = poison

    o_ext = lse_ext = None
    if n_ext:
        rows = total_q * H_q
        o_ext = np.empty((n_ext, rows, head_dim_v), np.float32)
        fill_normal(o_ext, kids["o_ext"])
        lse_ext = np.empty((n_ext, rows), np.float32)
        fill_normal(lse_ext, kids["lse_ext"], offset=ext_lse_center)
    return Workload(name=name, dtype=dtype, mla=mla, causal=causal, num_q_heads=H_q,
                    num_kv_heads=H_kv, head_dim_qk=head_dim_qk, head_dim_v=head_dim_v,
                    page_size=P, seq_lens=seq_lens.astype(np.int32),
                    q_lens=q_lens.astype(np.int32), page_table=table, num_pages=N, q=q,
                    k_pages=k_pages, v_pages=v_pages, scale=float(scale),
                    logical_to_physical=l2p, page_offsets=offsets.astype(np.int32),
                    n_ext=n_ext, o_ext=o_ext, lse_ext=lse_ext, chunk_tokens=chunk_tokens,
                    k_scale=k_scale, v_scale=v_scale)


# --------------------------------------------------------------------------------------
# The benchmark workloads. Lengths are drawn from the "lengths" stream. Workloads
# 1-5 are the five synthetic configurations; workload 6 adds a speculative-decoding
# step (LiquidCP section 7.1: 16 query tokens per request and iteration, one
# target token and 15 drafts) on a GQA group of 8, where the 16 tokens' rows
# make the products dense enough for the matrix cores; workload 7 is workload
# 2 over an FP8 E4M3 KV cache, workload 8 workload 3 over an FP8 E4M3 latent
# cache.
# --------------------------------------------------------------------------------------

MLA_DQK, MLA_DV, MLA_HEADS = 576, 512, 128
MLA_SCALE = 1.0 / math.sqrt(192.0)       # 1/sqrt(d_nope + d_rope) for DeepSeek-V3 dims
C3_SIGMA = math.sqrt(2.0 * math.log(12259.0 / 8192.0))
SHARP_GQA = 3.0                          # score std ~ 3 for N(0,1) q, k and scale 1/sqrt(D)
SHARP_MLA = 3.0 / (0.01 * math.sqrt(576.0) * MLA_SCALE)  # same for 0.1-scaled MLA values


def _lengths_rng(cid: int) -> np.random.Generator:
    kids = np.random.SeedSequence(SEED_BASE + cid).spawn(len(_STREAMS))
    return np.random.Generator(np.random.PCG64(kids[0]))


def config_lengths(cid: int):
    """(seq_lens, q_lens) of benchmark workload ``cid`` (1-based), before any shuffle."""
    if cid == 1:
        return np.array([100, 257]), np.array([1, 1])
    if cid == 2:
        L = _lengths_rng(2).integers(4096, 32768, size=32, endpoint=True)
        return L, np.ones(32, np.int64)
    if cid == 3:
        z = _lengths_rng(3).standard_normal(64)
        L = np.rint(np.exp(math.log(8192.0) + C3_SIGMA * z))
        return np.clip(L, 256, 131072).astype(np.int64), np.ones(64, np.int64)
    if cid == 4:
        short = _lengths_rng(4).integers(512, 2048, size=248, endpoint=True)
        L = np.concatenate([short, np.full(8, 262144)])
        return L, np.ones(256, np.int64)
    if cid == 5:
        L = np.array([1048576] * 8 + [65536 + 2048])
        n = np.array([1] * 8 + [2048])
        return L, n
    if cid == 6:
        L = _lengths_rng(6).integers(4096, 32768, size=32, endpoint=True)
        return L, np.full(32, 16, np.int64)
    if cid == 7:
        return config_lengths(2)
    if cid == 8:
        return config_lengths(3)
    raise ValueError(cid)


def make(cid: int, sharp: bool = False, decode_only: bool = False) -> Workload:
    """Benchmark workload ``cid`` (1..8). ``sharp`` scales q so that scores have a
    standard deviation of about 3 (a near-uniform softmax cannot reveal a wrong
    QK^T). ``decode_only`` (workload 5) drops the chunked-prefill request and the
    external states, leaving the eight million-token decode requests."""
    L, n = config_lengths(cid)
    seed = SEED_BASE + cid
    if cid == 1:
        return build("tiny-fp32-gqa", dtype="f32", mla=False, seq_lens=L, q_lens=n,
                     num_q_heads=4, num_kv_heads=1, head_dim_qk=64, head_dim_v=64,
                     page_size=16, scale=1.0 / 8.0, seed=seed, spare_pages=0,
                     q_scale=SHARP_GQA if sharp else 1.0, chunk_tokens=64)
    if cid == 2:
        return build("llama405b-gqa-share", dtype="bf16", mla=False, seq_lens=L, q_lens=n,
                     num_q_heads=128, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                     page_size=16, scale=1.0 / math.sqrt(128.0), seed=seed,
                     q_scale=SHARP_GQA if sharp else 1.0)
    if cid == 3:
        return build("deepseek-mla", dtype="bf16", mla=True, seq_lens=L, q_lens=n,
                     num_q_heads=MLA_HEADS, num_kv_heads=1, head_dim_qk=MLA_DQK,
                     head_dim_v=MLA_DV, page_size=64, scale=MLA_SCALE, seed=seed,
                     value_scale=0.1, q_scale=SHARP_MLA if sharp else 1.0)
    if cid == 4:
        return build("skewed-rollout-gqa", dtype="bf16", mla=False, seq_lens=L, q_lens=n,
                     num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                     page_size=16, scale=1.0 / math.sqrt(128.0), seed=seed, shuffle=True,
                     q_scale=SHARP_GQA if sharp else 1.0)
    if cid == 5:
        if decode_only:
            L, n = L[:8], n[:8]
        return build("mla-1m-shard" + ("-decode" if decode_only else ""), dtype="bf16",
                     mla=True, seq_lens=L, q_lens=n, num_q_heads=MLA_HEADS, num_kv_heads=1,
                     head_dim_qk=MLA_DQK, head_dim_v=MLA_DV, page_size=64, scale=MLA_SCALE,
                     seed=seed, value_scale=0.1, q_scale=SHARP_MLA if sharp else 1.0,
                     n_ext=0 if decode_only else 16,
                     ext_lse_center=math.log(1048576.0))
    if cid == 7:
        # workload 2's shape and lengths over an FP8 E4M3 KV cache
        return build("llama405b-gqa-share-fp8", dtype="fp8", mla=False, seq_lens=L, q_lens=n,
                     num_q_heads=128, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                     page_size=16, scale=1.0 / math.sqrt(128.0), seed=seed,
                     q_scale=SHARP_GQA if sharp else 1.0)
    if cid == 8:
        # workload 3's shape and lengths over an FP8 E4M3 latent cache (SPLASH
        # appendix C.1 serves its MLA backend from an FP8 E4M3 KV cache)
        return build("deepseek-mla-fp8", dtype="fp8", mla=True, seq_lens=L, q_lens=n,
                     num_q_heads=MLA_HEADS, num_kv_heads=1, head_dim_qk=MLA_DQK,
                     head_dim_v=MLA_DV, page_size=64, scale=MLA_SCALE, seed=seed,
                     value_scale=0.1, q_scale=SHARP_MLA if sharp else 1.0)
    if cid == 6:
        # causal rows: draft i sees the history and the tokens before it
        return build("spec-decode-gqa-g8", dtype="bf16", mla=False, seq_lens=L, q_lens=n,
                     num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                     page_size=16, scale=1.0 / math.sqrt(128.0), seed=seed,
                     q_scale=SHARP_GQA if sharp else 1.0)
    raise ValueError(cid)


def identity_layout(w: Workload) -> Workload:
    """The same logical KV with logical page i stored at physical page i (the
    spare pages follow). Results on it must equal results on ``w`` bit for bit."""
    n_used = w.logical_to_physical.shape[0]
    spare = np.setdiff1d(np.arange(w.num_pages, dtype=np.int32), w.logical_to_physical)
    src = np.concatenate([w.logical_to_physical, spare]).astype(np.int64)
    k = w.k_pages[src]
    v = None if w.v_pages is None else w.v_pages[src]
    ks = None if w.k_scale is None else w.k_scale[src]
    vs = None if w.v_scale is None else w.v_scale[src]
    pages_b = (w.seq_lens.astype(np.int64) + w.page_size - 1) // w.page_size
    table = np.full_like(w.page_table, n_used if spare.size else 0)
    for b in range(w.batch):
        table[b, : pages_b[b]] = np.arange(w.page_offsets[b], w.page_offsets[b + 1])
    out = Workload(**{**w.__dict__})
    out.k_pages, out.v_pages, out.page_table = k, v, table
    out.k_scale, out.v_scale = ks, vs
    out.logical_to_physical = np.arange(n_used, dtype=np.int32)
    out.name = w.name + "-identity"
    return out


def physical_slot(w: Workload, b: int, j: int):
    """(physical page, slot) holding logical token j of request b."""
    return int(w.page_table[b, j // w.page_size]), j % w.page_size


def set_logical_values(w: Workload, b: int, values: np.ndarray) -> None:
    """Store logical values [L_b][H_kv][D_v] of request b into its pages (GQA:
    v_pages; MLA: the first D_v columns of the latent rows). Layout only."""
    assert w.dtype != "fp8", "values of an fp8 cache are codes with scales"
    P = w.page_size
    L = int(w.seq_lens[b])
    for p in range((L + P - 1) // P):
        pid = int(w.page_table[b, p])
        lo, hi = p * P, min(L, (p + 1) * P)
        blk = values[lo:hi]                      # [t][H_kv][D_v]
        if w.mla:
            w.k_pages[pid, : hi - lo, : w.head_dim_v] = blk[:, 0, :]
        else:
            w.v_pages[pid, :, :, : hi - lo] = np.transpose(blk, (1, 2, 0))


def zero_keys(w: Workload) -> None:
    """Set every key to zero (GQA: all of k_pages; MLA: all 576 columns), keeping
    the poison of unused slots. Layout only."""
    zero = {"bf16": np.uint16(0), "fp8": np.uint8(0)}.get(w.dtype, np.float32(0))
    P = w.page_size
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for p in range((L + P - 1) // P):
            pid = int(w.page_table[b, p])
            used = min(P, L - p * P)
            if w.mla:
                w.k_pages[pid, :used, :] = zero
            else:
                w.k_pages[pid, :, :, :used, :] = zero
