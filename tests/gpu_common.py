"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C ABI, and compare with the float64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import split_kv_partial_amd as skv
from oracle import attention as A

TOL_F32 = dict(abs=1e-5, rel=1e-5, lse=1e-5)
TOL_BF16 = dict(abs=2e-3, rel=1e-2, lse=2e-3)


def tol_for(w):
    """fp32 storage: 1e-5; bf16 storage and FP8 KV (bf16 queries, codes decoded
    exactly to bf16, the same bf16 products with fp32 accumulation): the bf16
    bound."""
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def spec_of(w) -> skv.AttnSpec:
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": skv.FP8}[w.dtype]
    return skv.AttnSpec(w.num_q_heads, w.num_kv_heads, w.head_dim_qk, w.head_dim_v, w.page_size,
                        dtype=dt, mla=w.mla, causal=w.causal)


def _dev_tensor(a: np.ndarray, dtype: str, dev):
    """bf16 bits (uint16) as a bf16 tensor; float32 and fp8 codes (uint8) as they are."""
    if dtype == "bf16" or (dtype == "fp8" and a.dtype == np.uint16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class DeviceInputs:
    def __init__(self, w, dev="cuda:0"):
        self.q = _dev_tensor(w.q, w.dtype, dev)
        self.k = _dev_tensor(w.k_pages, w.dtype, dev)
        self.v = self.k if w.mla else _dev_tensor(w.v_pages, w.dtype, dev)
        self.k_scale = None if w.k_scale is None else torch.from_numpy(w.k_scale).to(dev)
        # FP8 MLA rows: one scale per page for keys and values (the same tensor)
        self.v_scale = (self.k_scale if w.mla else
                        None if w.v_scale is None else torch.from_numpy(w.v_scale).to(dev))
        self.page_table = torch.from_numpy(w.page_table).to(dev)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(dev)
        self.o_ext = None if w.o_ext is None else torch.from_numpy(w.o_ext).to(dev)
        self.lse_ext = None if w.lse_ext is None else torch.from_numpy(w.lse_ext).to(dev)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def run_path(w, plan, inputs: DeviceInputs | None = None, with_ext: bool = True,
             out_dtype=torch.float32, fused: bool = True):
    """Partial states and merged output of the HIP path (the two calls), as
    float64 numpy arrays. With ``fused``, the one-call path (attention and
    merge in one launch for plans built for it, else the two launches; FP8 KV
    through its own one-call entry point) also runs on the same inputs and
    must give the same merged output and LSE bit for bit: both merges add a
    row's states in the same order with the same operations."""
    d = inputs or DeviceInputs(w)
    fp8 = w.dtype == "fp8"
    if fp8:
        # FP8 KV has its own entry points (with the scales); its one-call path
        # runs the two launches
        o_part, lse_part = skv.decode_attn_partial_fp8(d.q, d.k, d.v, d.k_scale, d.v_scale, d.page_table,
                                                       d.seq_lens, plan, w.scale)
    else:
        o_part, lse_part = skv.decode_attn_partial(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale)
    ext = with_ext and d.o_ext is not None
    o, lse = skv.merge_states(o_part, lse_part, plan, d.o_ext if ext else None,
                              d.lse_ext if ext else None, out_dtype=out_dtype)
    if fused and fp8:
        fo, fl = skv.decode_attn_fp8(d.q, d.k, d.v, d.k_scale, d.v_scale, d.page_table, d.seq_lens, plan,
                                     w.scale, d.o_ext if ext else None, d.lse_ext if ext else None,
                                     out_dtype=out_dtype)
    elif fused:
        fo, fl = skv.decode_attn(d.q, d.k, d.v, d.page_table, d.seq_lens, plan, w.scale,
                                 d.o_ext if ext else None, d.lse_ext if ext else None,
                                 out_dtype=out_dtype)
    if fused:
        torch.cuda.synchronize()
        assert torch.equal(_bits(fo), _bits(o)), f"{w.name}: fused output differs from the two calls"
        assert torch.equal(_bits(fl), _bits(lse)), f"{w.name}: fused LSE differs from the two calls"
    torch.cuda.synchronize()
    return (o_part.cpu().double().numpy(), lse_part.cpu().double().numpy(),
            o.float().cpu().double().numpy(), lse.cpu().double().numpy())


def compare(o_gpu, o_ref, l_gpu, l_ref, tol, what=""):
    """Element-wise comparison: max abs and relative L2 on O, max abs on LSE;
    rows the oracle marks empty (LSE = -inf) must be exactly (0, -inf)."""
    o_gpu = np.asarray(o_gpu, np.float64).reshape(o_ref.shape)
    l_gpu = np.asarray(l_gpu, np.float64).reshape(l_ref.shape)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), empty), f"{what}: empty-state pattern differs"
    assert np.all(o_gpu[empty] == 0), f"{what}: empty states must hold O = 0"
    ok = ~empty
    assert np.isfinite(o_gpu[ok]).all() and np.isfinite(l_gpu[ok]).all(), f"{what}: non-finite output"
    err = np.abs(o_gpu[ok] - o_ref[ok])
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(o_ref[ok])) or 1.0
    rel = float(np.linalg.norm(o_gpu[ok] - o_ref[ok])) / denom
    lerr = float(np.max(np.abs(l_gpu[ok] - l_ref[ok]))) if ok.any() else 0.0
    msg = f"{what}: max|dO|={max_abs:.3g} relL2={rel:.3g} max|dLSE|={lerr:.3g}"
    assert max_abs <= tol["abs"] and rel <= tol["rel"] and lerr <= tol["lse"], msg
    return max_abs, rel, lerr


def oracle_partials(w, plan, requests=None, token_ids=None):
    """Oracle partial states laid out like the plan's o_part / lse_part rows.

    Returns dict b -> (O [s][n][H][D_v], LSE [s][n][H]) for the listed requests."""
    out = {}
    ranges = plan.ranges()
    for b in (range(w.batch) if requests is None else requests):
        ids = None if token_ids is None else token_ids[b]
        out[b] = A.partial_states(w, b, ranges[b], token_ids=ids)
    return out


def gpu_partials_of(w, plan, o_part, lse_part, b, token_ids=None):
    """The plan's o_part / lse_part rows of request b as [s][n][H][D_v] / [s][n][H]."""
    e = plan.export()
    s = int(e["split_counts"][b])
    off = int(e["state_row_offset"][b])
    n = int(w.q_lens[b])
    H = w.num_q_heads
    o = o_part[off: off + s * n * H].reshape(s, n, H, -1)
    l = lse_part[off: off + s * n * H].reshape(s, n, H)
    if token_ids is not None:
        o, l = o[:, token_ids], l[:, token_ids]
    return o, l


def check_all(w, plan, inputs=None, check_partials=True, token_ids=None, requests=None):
    """Run the HIP path and compare every (or the listed) row's partial states and
    merged output with the oracle."""
    tol = tol_for(w)
    o_part, lse_part, o, lse = run_path(w, plan, inputs)
    reqs = range(w.batch) if requests is None else requests
    qoff = A.q_offsets(w)
    H = w.num_q_heads
    ref_parts = oracle_partials(w, plan, reqs, token_ids) if check_partials else None
    for b in reqs:
        ids = list(range(int(w.q_lens[b]))) if token_ids is None else list(token_ids[b])
        if check_partials:
            go, gl = gpu_partials_of(w, plan, o_part, lse_part, b, ids if token_ids is not None else None)
            ro, rl = ref_parts[b]
            compare(go, ro, gl, rl, tol, f"{w.name} partial b={b}")
        ref_o, ref_l = A.attention_rows(w, b, ids)
        if w.n_ext and w.o_ext is not None:
            rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
            eo = w.o_ext[:, rows].reshape(w.n_ext, len(ids), H, -1).astype(np.float64)
            el = w.lse_ext[:, rows].reshape(w.n_ext, len(ids), H).astype(np.float64)
            ref_o, ref_l = A.merge(np.concatenate([ref_o[None], eo]), np.concatenate([ref_l[None], el]))
        rows = np.array([(qoff[b] + i) * H + h for i in ids for h in range(H)])
        compare(o[rows].reshape(ref_o.shape), ref_o, lse[rows].reshape(ref_l.shape), ref_l, tol,
                f"{w.name} merged b={b}")
    return o_part, lse_part, o, lse
