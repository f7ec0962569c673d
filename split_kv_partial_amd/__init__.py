"""Split-KV partial decode attention for AMD MI355X (gfx950).

Python face of ``libsplitkv.so``: argument marshalling only. Planning runs in
the library's C++ planner and every step of the attention and merge runs in its
HIP kernels; torch supplies device memory and streams. Importing this module
without the built library raises ``ImportError`` (build it with
``python split_kv_partial_amd/build.py``).

    spec = AttnSpec(num_q_heads=128, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                    page_size=16, dtype=torch.bfloat16)
    plan = plan_splits(seq_lens, spec, num_cu=256)
    o_part, lse_part = decode_attn_partial(q, k_pages, v_pages, page_table, seq_lens_dev,
                                           plan, scale)
    o, lse = merge_states(o_part, lse_part, plan)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SKV_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("SKV_LIBRARY") or os.path.join(_HERE, "libsplitkv.so")

SKV_F32, SKV_BF16, SKV_FP8_E4M3 = 0, 1, 2
# AttnSpec dtype of an FP8 KV cache: bf16 queries, E4M3 keys and values
FP8 = torch.float8_e4m3fn
STATUS = {0: "SKV_OK", -1: "SKV_ERR_INVALID_ARG", -2: "SKV_ERR_UNSUPPORTED", -3: "SKV_ERR_HIP",
          -4: "SKV_ERR_NO_MEMORY", -5: "SKV_ERR_PLAN_MISMATCH"}

# Every symbol the public header declares.
EXPORTED = (
    "skv_plan_params_default", "skv_plan_splits", "skv_plan_from_counts", "skv_plan_fixed_chunks",
    "skv_plan_get_info", "skv_plan_export", "skv_plan_workspace_bytes", "skv_plan_upload",
    "skv_plan_destroy", "skv_decode_attn_partial", "skv_merge_states", "skv_read_error_flag",
    "skv_hbm_read_probe", "skv_last_error", "skv_decode_attn_scratch_bytes", "skv_decode_attn",
    "skv_decode_attn_noalloc", "skv_decode_attn_partial_fp8", "skv_mfma_probe", "skv_decode_attn_fp8",
)


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("mla", ctypes.c_int32), ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class PlanParams(ctypes.Structure):
    _fields_ = [("tile_tokens", ctypes.c_int32), ("slots_per_cu", ctypes.c_int32),
                ("warps_per_slot", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("overlap_reduction", ctypes.c_int32), ("use_calibration", ctypes.c_int32),
                ("balanced_candidates", ctypes.c_int32), ("query_tile", ctypes.c_int32),
                ("rho", ctypes.c_double), ("delta_attn", ctypes.c_double),
                ("delta_red", ctypes.c_double), ("gamma", ctypes.c_double),
                ("min_gain", ctypes.c_double), ("tile_time_us", ctypes.c_double)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_tasks", ctypes.c_int32),
                ("total_splits", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("warps_per_slot", ctypes.c_int32), ("reduction_run", ctypes.c_int32),
                ("num_units", ctypes.c_int32), ("split_adopted", ctypes.c_int32),
                ("state_rows", ctypes.c_int64), ("total_rows", ctypes.c_int64),
                ("score", ctypes.c_double), ("t_attn", ctypes.c_double),
                ("nosplit_score", ctypes.c_double), ("rho", ctypes.c_double),
                ("delta_attn", ctypes.c_double), ("delta_red", ctypes.c_double),
                ("gamma", ctypes.c_double), ("tile_time_us", ctypes.c_double),
                ("balanced_candidates", ctypes.c_int32), ("query_tile", ctypes.c_int32),
                ("reference_score", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python split_kv_partial_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    pdesc = ctypes.POINTER(AttnDesc)
    pprm = ctypes.POINTER(PlanParams)
    pplan = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "skv_plan_params_default": (None, [pprm]),
        "skv_plan_splits": (I32, [pdesc, pi32, pi32, I32, I32, pprm, pi32, pplan]),
        "skv_plan_from_counts": (I32, [pdesc, pi32, pi32, pi32, I32, I32, pprm, pplan]),
        "skv_plan_fixed_chunks": (I32, [pdesc, pi32, pi32, I32, I32, pplan]),
        "skv_plan_get_info": (I32, [P, ctypes.POINTER(PlanInfo)]),
        "skv_plan_export": (I32, [P, pi32, pi32, pi32, pi64, pi32]),
        "skv_plan_workspace_bytes": (SZ, [P]),
        "skv_plan_upload": (I32, [P, P, SZ, P]),
        "skv_plan_destroy": (None, [P]),
        "skv_decode_attn_partial": (I32, [pdesc, P, P, P, P, P, P, P, P, P, P]),
        "skv_decode_attn_partial_fp8": (I32, [pdesc, P, P, P, P, P, P, P, P, P, P, P, P]),
        "skv_merge_states": (I32, [pdesc, P, P, P, P, I32, P, P, P, I32, P, P]),
        "skv_decode_attn_scratch_bytes": (SZ, [P]),
        "skv_decode_attn": (I32, [pdesc, P, P, P, P, P, P, P, P, SZ, I32, P, P, P, I32, P, P]),
        "skv_decode_attn_noalloc": (I32, [pdesc, P, P, P, P, P, P, P, I32, P, P, P, I32, P, P]),
        "skv_decode_attn_fp8": (I32, [pdesc, P, P, P, P, P, P, P, P, P, P, SZ, I32, P, P, P, I32, P, P]),
        "skv_read_error_flag": (I32, [P, pi32, P]),
        "skv_hbm_read_probe": (I32, [P, I64, P, I32, P]),
        "skv_mfma_probe": (I32, [P, I64, I32, P, I32, I32, I32, I32, P]),
        "skv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


class SplitKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.skv_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise SplitKVError(status, where)


def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


@dataclass
class AttnSpec:
    """Shape of an attention layer (everything but the batch's lengths)."""
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    dtype: torch.dtype = torch.bfloat16
    mla: bool = False
    causal: bool = True

    def desc(self, batch: int, max_pages: int = 1, num_pages: int = 1, scale: float = 1.0) -> AttnDesc:
        code = {torch.bfloat16: SKV_BF16, torch.float32: SKV_F32, FP8: SKV_FP8_E4M3}[self.dtype]
        return AttnDesc(batch, self.num_q_heads, self.num_kv_heads, self.head_dim_qk, self.head_dim_v,
                        self.page_size, max_pages, num_pages, int(self.mla), int(self.causal), code,
                        float(scale))

    @property
    def q_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == FP8 else self.dtype

    @property
    def kv_dtypes(self) -> tuple:
        return (torch.uint8, FP8) if self.dtype == FP8 else (self.dtype,)


def default_params() -> PlanParams:
    p = PlanParams()
    _lib.skv_plan_params_default(ctypes.byref(p))
    return p


class Plan:
    """Owns a host plan; uploads its descriptors to a device workspace on demand."""

    def __init__(self, handle: ctypes.c_void_p, spec: AttnSpec, seq_lens, q_lens):
        self._h = handle
        self.spec = spec
        self.seq_lens = np.asarray(seq_lens, np.int64).copy()
        self.q_lens = np.asarray(q_lens, np.int64).copy()
        self.max_pages = int(((self.seq_lens + spec.page_size - 1) // spec.page_size).max())
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            for ws, ev in self._ws.values():
                ev.synchronize()     # the upload reads host memory the plan owns
            _lib.skv_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def info(self) -> PlanInfo:
        inf = PlanInfo()
        _check(_lib.skv_plan_get_info(self._h, ctypes.byref(inf)), "skv_plan_get_info")
        return inf

    def export(self) -> dict:
        inf = self.info()
        B = inf.batch
        counts = np.zeros(B, np.int32)
        start = np.zeros(max(1, inf.total_splits), np.int32)
        end = np.zeros(max(1, inf.total_splits), np.int32)
        off = np.zeros(B + 1, np.int64)
        order = np.zeros((max(1, inf.num_tasks), 4), np.int32)
        p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        _check(_lib.skv_plan_export(self._h, p32(counts), p32(start), p32(end),
                                    off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), p32(order)),
               "skv_plan_export")
        return {"split_counts": counts, "split_start": start[: inf.total_splits],
                "split_end": end[: inf.total_splits], "state_row_offset": off,
                "task_order": order[: inf.num_tasks]}

    def ranges(self):
        """Per request, the list of (start, end) token ranges of its splits."""
        e = self.export()
        out, k = [], 0
        for c in e["split_counts"]:
            out.append(list(zip(e["split_start"][k:k + c].tolist(), e["split_end"][k:k + c].tolist())))
            k += c
        return out

    def workspace_bytes(self) -> int:
        return int(_lib.skv_plan_workspace_bytes(self._h))

    def workspace(self, device=None) -> torch.Tensor:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        key = dev.index
        if key not in self._ws:
            n = self.workspace_bytes()
            ws = torch.empty(n, dtype=torch.uint8, device=dev)
            with torch.cuda.device(dev):
                _check(_lib.skv_plan_upload(self._h, ws.data_ptr(), n, _stream_ptr()), "skv_plan_upload")
                ev = torch.cuda.Event()
                ev.record()
            self._ws[key] = (ws, ev)
        return self._ws[key][0]

    def read_error_flag(self, device=None) -> int:
        ws = self.workspace(device)
        flag = ctypes.c_int32(0)
        _check(_lib.skv_read_error_flag(ws.data_ptr(), ctypes.byref(flag), _stream_ptr()),
               "skv_read_error_flag")
        return flag.value


def _make_plan(fn_name, spec, seq_lens, q_lens, *extra):
    L, Lp = _i32(seq_lens)
    B = L.shape[0]
    if q_lens is None:
        q_lens = np.ones(B, np.int32)
    n, npp = _i32(q_lens)
    max_pages = int(((L.astype(np.int64) + spec.page_size - 1) // spec.page_size).max())
    desc = spec.desc(B, max_pages=max_pages, num_pages=1)
    h = ctypes.c_void_p()
    _check(getattr(_lib, fn_name)(ctypes.byref(desc), Lp, npp, *extra, ctypes.byref(h)), fn_name)
    return Plan(h, spec, L, n)


def plan_splits(seq_lens, spec: AttnSpec, num_cu: int = 256, q_lens=None, n_ext: int = 0,
                params: PlanParams | None = None, ref_splits=None) -> Plan:
    """Critical-wave split plan for a batch (host planner, once per batch)."""
    ref = None
    if ref_splits is not None:
        ref_arr, ref = _i32(ref_splits)
    return _make_plan("skv_plan_splits", spec, seq_lens, q_lens, int(num_cu), int(n_ext),
                      None if params is None else ctypes.byref(params), ref)


def plan_from_counts(seq_lens, spec: AttnSpec, split_counts, num_cu: int = 256, q_lens=None,
                     n_ext: int = 0, params: PlanParams | None = None) -> Plan:
    cnt, cp = _i32(split_counts)
    return _make_plan("skv_plan_from_counts", spec, seq_lens, q_lens, cp, int(num_cu), int(n_ext),
                      None if params is None else ctypes.byref(params))


def plan_fixed_chunks(seq_lens, spec: AttnSpec, chunk_tokens: int, num_cu: int = 256,
                      q_lens=None) -> Plan:
    return _make_plan("skv_plan_fixed_chunks", spec, seq_lens, q_lens, int(chunk_tokens), int(num_cu))


def _check_tensor(t, name: str, dev, dtypes, numel=None, shape=None) -> None:
    """Raise ValueError unless t is a contiguous tensor on dev with one of
    dtypes and, when given, exactly `shape` or at least `numel` elements. The
    C ABI takes bare device pointers, so buffer sizes are checked here."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not t.is_contiguous() or t.device != dev:
        raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")


def _desc_for(plan: Plan, page_table: torch.Tensor, k_pages: torch.Tensor, scale: float) -> AttnDesc:
    return plan.spec.desc(len(plan.seq_lens), max_pages=page_table.shape[1],
                          num_pages=k_pages.shape[0], scale=scale)


def _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan: Plan) -> None:
    sp = plan.spec
    dev = q.device
    B = len(plan.seq_lens)
    _check_tensor(q, "q", dev, (sp.q_dtype,),
                  shape=(int(plan.q_lens.sum()), sp.num_q_heads, sp.head_dim_qk))
    _check_tensor(k_pages, "k_pages", dev, sp.kv_dtypes)
    if k_pages.dim() < 1 or k_pages.shape[0] < 1:
        raise ValueError("k_pages must hold at least one page")
    n_pages = int(k_pages.shape[0])
    if sp.mla:
        if v_pages is not k_pages and v_pages.data_ptr() != k_pages.data_ptr():
            raise ValueError("MLA reads values from the key rows: v_pages must be k_pages")
        if k_pages.numel() != n_pages * sp.page_size * sp.head_dim_qk:
            raise ValueError(f"MLA k_pages must be [num_pages][{sp.page_size}][{sp.head_dim_qk}]")
    else:
        per_page_k = sp.num_kv_heads * sp.head_dim_qk * sp.page_size
        per_page_v = sp.num_kv_heads * sp.head_dim_v * sp.page_size
        if k_pages.numel() != n_pages * per_page_k:
            raise ValueError(f"k_pages must hold {per_page_k} elements per page")
        _check_tensor(v_pages, "v_pages", dev, sp.kv_dtypes, numel=n_pages * per_page_v)
    _check_tensor(page_table, "page_table", dev, (torch.int32,))
    if page_table.dim() != 2 or page_table.shape[0] != B or page_table.shape[1] < plan.max_pages:
        raise ValueError(f"page_table must be [{B}][>= {plan.max_pages}] int32, "
                         f"got {tuple(page_table.shape)}")
    _check_tensor(seq_lens, "seq_lens", dev, (torch.int32,), shape=(B,))


def _merge_outputs(plan: Plan, dev, o_ext, lse_ext, out_dtype, o_out, lse_out, want_lse):
    """Checked (n_ext, o_out, lse_out) of a merge; outputs allocated when not given."""
    inf = plan.info()
    dv = plan.spec.head_dim_v
    if (o_ext is None) != (lse_ext is None):
        raise ValueError("o_ext and lse_ext go together")
    n_ext = 0 if o_ext is None else int(o_ext.shape[0])
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    if o_out is None:
        o_out = torch.empty(inf.total_rows, dv, dtype=out_dtype, device=dev)
    if want_lse and lse_out is None:
        lse_out = torch.empty(inf.total_rows, dtype=torch.float32, device=dev)
    if o_ext is not None:
        _check_tensor(o_ext, "o_ext", dev, (torch.float32,), shape=(n_ext, inf.total_rows, dv))
        _check_tensor(lse_ext, "lse_ext", dev, (torch.float32,), shape=(n_ext, inf.total_rows))
    _check_tensor(o_out, "o_out", dev, (torch.float32, torch.bfloat16), numel=inf.total_rows * dv)
    if lse_out is not None:
        _check_tensor(lse_out, "lse_out", dev, (torch.float32,), numel=inf.total_rows)
    return n_ext, o_out, lse_out


def _out_dtype_code(o_out) -> int:
    return SKV_BF16 if o_out.dtype == torch.bfloat16 else SKV_F32


def decode_attn_partial(q, k_pages, v_pages, page_table, seq_lens, plan: Plan, scale: float,
                        o_part=None, lse_part=None):
    """Partial states (O_r normalised over split r, natural-log LSE_r) for every
    split of ``plan``. Returns (o_part [state_rows][D_v], lse_part [state_rows])."""
    inf = plan.info()
    sp = plan.spec
    dev = q.device
    if sp.dtype == FP8:
        raise ValueError("an FP8 KV cache needs its scales: use decode_attn_partial_fp8")
    if o_part is None:
        o_part = torch.empty(inf.state_rows, sp.head_dim_v, dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty(inf.state_rows, dtype=torch.float32, device=dev)
    _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan)
    _check_tensor(o_part, "o_part", dev, (torch.float32,), numel=inf.state_rows * sp.head_dim_v)
    _check_tensor(lse_part, "lse_part", dev, (torch.float32,), numel=inf.state_rows)
    desc = _desc_for(plan, page_table, k_pages, scale)
    ws = plan.workspace(dev)
    _check(_lib.skv_decode_attn_partial(ctypes.byref(desc), q.data_ptr(), k_pages.data_ptr(),
                                        v_pages.data_ptr(), page_table.data_ptr(), seq_lens.data_ptr(),
                                        plan.handle, ws.data_ptr(), o_part.data_ptr(),
                                        lse_part.data_ptr(), _stream_ptr()),
           "skv_decode_attn_partial")
    return o_part, lse_part



def decode_attn_partial_fp8(q, k_pages, v_pages, k_scales, v_scales, page_table, seq_lens, plan: Plan,
                            scale: float, o_part=None, lse_part=None):
    """decode_attn_partial over an FP8 (OCP E4M3) KV cache: k_pages / v_pages
    hold codes (uint8 or float8_e4m3fn) in the GQA layouts with X = 16, or MLA
    rows [num_pages][P][576] (v_pages is k_pages), and k_scales / v_scales
    [num_pages][H_kv] float32 the per-page, per-KV-head factors of the decoded
    keys and values (MLA: one scale per page, v_scales is k_scales). The plan's
    spec has dtype FP8."""
    inf = plan.info()
    sp = plan.spec
    dev = q.device
    if sp.dtype != FP8:
        raise ValueError("decode_attn_partial_fp8 needs a plan built for dtype FP8")
    if o_part is None:
        o_part = torch.empty(inf.state_rows, sp.head_dim_v, dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty(inf.state_rows, dtype=torch.float32, device=dev)
    _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan)
    n_pages = int(k_pages.shape[0])
    _check_tensor(k_scales, "k_scales", dev, (torch.float32,), shape=(n_pages, sp.num_kv_heads))
    _check_tensor(v_scales, "v_scales", dev, (torch.float32,), shape=(n_pages, sp.num_kv_heads))
    if sp.mla and v_scales.data_ptr() != k_scales.data_ptr():
        raise ValueError("FP8 MLA rows have one scale per page: v_scales must be k_scales")
    _check_tensor(o_part, "o_part", dev, (torch.float32,), numel=inf.state_rows * sp.head_dim_v)
    _check_tensor(lse_part, "lse_part", dev, (torch.float32,), numel=inf.state_rows)
    desc = _desc_for(plan, page_table, k_pages, scale)
    ws = plan.workspace(dev)
    _check(_lib.skv_decode_attn_partial_fp8(ctypes.byref(desc), q.data_ptr(), k_pages.data_ptr(),
                                            v_pages.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(),
                                            page_table.data_ptr(), seq_lens.data_ptr(), plan.handle,
                                            ws.data_ptr(), o_part.data_ptr(), lse_part.data_ptr(),
                                            _stream_ptr()),
           "skv_decode_attn_partial_fp8")
    return o_part, lse_part


def merge_states(o_part, lse_part, plan: Plan, o_ext=None, lse_ext=None,
                 out_dtype=torch.float32, o_out=None, lse_out=None, want_lse: bool = True):
    """Exact LSE merge of each row's local splits plus optional external states
    (o_ext [n_ext][total_rows][D_v], lse_ext [n_ext][total_rows], float32).
    Returns (O [total_rows][D_v], LSE [total_rows] or None)."""
    inf = plan.info()
    dv = plan.spec.head_dim_v
    dev = o_part.device
    n_ext, o_out, lse_out = _merge_outputs(plan, dev, o_ext, lse_ext, out_dtype, o_out, lse_out, want_lse)
    _check_tensor(o_part, "o_part", dev, (torch.float32,), numel=inf.state_rows * dv)
    _check_tensor(lse_part, "lse_part", dev, (torch.float32,), numel=inf.state_rows)
    desc = plan.spec.desc(len(plan.seq_lens), max_pages=plan.max_pages, num_pages=1)
    ws = plan.workspace(dev)
    _check(_lib.skv_merge_states(ctypes.byref(desc), plan.handle, ws.data_ptr(), o_part.data_ptr(),
                                 lse_part.data_ptr(), n_ext, _ptr(o_ext), _ptr(lse_ext),
                                 o_out.data_ptr(), _out_dtype_code(o_out), _ptr(lse_out), _stream_ptr()),
           "skv_merge_states")
    return o_out, lse_out


def scratch_bytes(plan: Plan) -> int:
    """Device scratch bytes decode_attn needs for ``plan``."""
    return int(_lib.skv_decode_attn_scratch_bytes(plan.handle))


def decode_attn(q, k_pages, v_pages, page_table, seq_lens, plan: Plan, scale: float,
                o_ext=None, lse_ext=None, out_dtype=torch.float32, o_out=None, lse_out=None,
                want_lse: bool = True, scratch=None):
    """The whole path in one library call: partial states of every split into
    ``scratch`` (a uint8 device tensor of at least scratch_bytes(plan) bytes;
    allocated when not given), then their merge with optional external states.
    Returns (O [total_rows][D_v], LSE [total_rows] or None)."""
    dev = q.device
    _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan)
    n_ext, o_out, lse_out = _merge_outputs(plan, dev, o_ext, lse_ext, out_dtype, o_out, lse_out, want_lse)
    need = scratch_bytes(plan)
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_tensor(scratch, "scratch", dev, (torch.uint8,), numel=need)
    desc = _desc_for(plan, page_table, k_pages, scale)
    ws = plan.workspace(dev)
    _check(_lib.skv_decode_attn(ctypes.byref(desc), q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                page_table.data_ptr(), seq_lens.data_ptr(), plan.handle, ws.data_ptr(),
                                scratch.data_ptr(), scratch.numel(), n_ext, _ptr(o_ext), _ptr(lse_ext),
                                o_out.data_ptr(), _out_dtype_code(o_out), _ptr(lse_out), _stream_ptr()),
           "skv_decode_attn")
    return o_out, lse_out


def decode_attn_fp8(q, k_pages, v_pages, k_scales, v_scales, page_table, seq_lens, plan: Plan, scale: float,
                    o_ext=None, lse_ext=None, out_dtype=torch.float32, o_out=None, lse_out=None,
                    want_lse: bool = True, scratch=None):
    """decode_attn over an FP8 (OCP E4M3) KV cache, with the scales of
    decode_attn_partial_fp8; the plan is built for dtype FP8 with
    overlap_reduction = 0 (the two launches)."""
    dev = q.device
    sp = plan.spec
    if sp.dtype != FP8:
        raise ValueError("decode_attn_fp8 needs a plan built for dtype FP8")
    _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan)
    n_pages = int(k_pages.shape[0])
    _check_tensor(k_scales, "k_scales", dev, (torch.float32,), shape=(n_pages, sp.num_kv_heads))
    _check_tensor(v_scales, "v_scales", dev, (torch.float32,), shape=(n_pages, sp.num_kv_heads))
    if sp.mla and v_scales.data_ptr() != k_scales.data_ptr():
        raise ValueError("FP8 MLA rows have one scale per page: v_scales must be k_scales")
    n_ext, o_out, lse_out = _merge_outputs(plan, dev, o_ext, lse_ext, out_dtype, o_out, lse_out, want_lse)
    need = scratch_bytes(plan)
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_tensor(scratch, "scratch", dev, (torch.uint8,), numel=need)
    desc = _desc_for(plan, page_table, k_pages, scale)
    ws = plan.workspace(dev)
    _check(_lib.skv_decode_attn_fp8(ctypes.byref(desc), q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                    k_scales.data_ptr(), v_scales.data_ptr(), page_table.data_ptr(),
                                    seq_lens.data_ptr(), plan.handle, ws.data_ptr(), scratch.data_ptr(),
                                    scratch.numel(), n_ext, _ptr(o_ext), _ptr(lse_ext), o_out.data_ptr(),
                                    _out_dtype_code(o_out), _ptr(lse_out), _stream_ptr()),
           "skv_decode_attn_fp8")
    return o_out, lse_out


NOALLOC_SCRATCH_BYTES = 128 << 20   # the library's per-device scratch array


def decode_attn_noalloc(q, k_pages, v_pages, page_table, seq_lens, plan: Plan, scale: float,
                        o_ext=None, lse_ext=None, out_dtype=torch.float32, o_out=None, lse_out=None,
                        want_lse: bool = True):
    """decode_attn with the partial states in the library's per-device scratch
    array (no device allocation inside the call; o_out / lse_out are
    allocated here only when not given). Plans needing more than
    NOALLOC_SCRATCH_BYTES raise; calls overlapping on one device race."""
    dev = q.device
    _check_attention_inputs(q, k_pages, v_pages, page_table, seq_lens, plan)
    n_ext, o_out, lse_out = _merge_outputs(plan, dev, o_ext, lse_ext, out_dtype, o_out, lse_out, want_lse)
    desc = _desc_for(plan, page_table, k_pages, scale)
    ws = plan.workspace(dev)
    _check(_lib.skv_decode_attn_noalloc(ctypes.byref(desc), q.data_ptr(), k_pages.data_ptr(),
                                        v_pages.data_ptr(), page_table.data_ptr(), seq_lens.data_ptr(),
                                        plan.handle, ws.data_ptr(), n_ext, _ptr(o_ext), _ptr(lse_ext),
                                        o_out.data_ptr(), _out_dtype_code(o_out), _ptr(lse_out),
                                        _stream_ptr()),
           "skv_decode_attn_noalloc")
    return o_out, lse_out


def hbm_read_probe(buf: torch.Tensor, blocks: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Streaming read of the contiguous device tensor `buf` (a measurement
    utility for the HBM read ceiling, not a step of the method); returns
    out [blocks] uint32-valued int32, whose XOR is the XOR of buf's words."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf must be a contiguous device tensor")
    if out is None:
        out = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    _check(_lib.skv_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                   int(blocks), _stream_ptr()),
           "skv_hbm_read_probe")
    return out


def mfma_probe(blocks: int, waves: int, iters: int, device, out: torch.Tensor | None = None,
               mfma_waves: int | None = None, buf: torch.Tensor | None = None, passes: int = 0) -> torch.Tensor:
    """Dense bf16 matrix-core load, optionally beside an HBM stream (a
    measurement utility for the sustained matrix rate, not a step of the
    method): `blocks` work-groups of `waves` waves; the first `mfma_waves`
    (default: all) run 8 * iters products of 16x16x32 each, the others read
    the contiguous device tensor `buf` `passes` times. Returns out
    [blocks * waves, 2] int32: per wave a word folded from its results and the
    shader-clock cycles of its loop."""
    mw = waves if mfma_waves is None else mfma_waves
    if out is None:
        out = torch.empty(blocks * waves, 2, dtype=torch.int32, device=device)
    if (out.dtype != torch.int32 or out.device.type != "cuda" or not out.is_contiguous()
            or out.numel() < 2 * blocks * waves):
        raise ValueError("out must be a contiguous device tensor of 2 * blocks * waves int32")
    if mw < waves and (buf is None or not buf.is_contiguous() or buf.device.type != "cuda"):
        raise ValueError("streaming waves need buf, a contiguous device tensor")
    ptr, nbytes = (buf.data_ptr(), buf.numel() * buf.element_size()) if buf is not None else (None, 0)
    _check(_lib.skv_mfma_probe(ptr, nbytes, int(passes), out.data_ptr(), int(blocks), int(waves), int(mw),
                               int(iters), _stream_ptr()),
           "skv_mfma_probe")
    return out
