"""C ABI checks that need no GPU: the library loads, exports every symbol the
public header declares, and rejects bad arguments with the documented status
codes before anything is enqueued."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

import split_kv_partial_amd as skv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitkv.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 13
    lib = ctypes.CDLL(skv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(skv.EXPORTED) == names


def test_defaults_are_the_papers_table2():
    p = skv.default_params()
    assert (p.rho, p.delta_attn, p.delta_red, p.gamma) == (0.43, 32.0, 2.5, 0.47)
    assert p.tile_tokens == 64 and p.max_splits == 64 and abs(p.min_gain - 0.10) < 1e-15
    assert p.use_calibration == 1


def test_calibration_switch():
    spec = skv.AttnSpec(128, 8, 128, 128, 16)
    p = skv.default_params()
    p.use_calibration = 0
    inf = skv.plan_splits([5000, 7000], spec, 8, params=p).info()
    assert (inf.rho, inf.delta_attn, inf.delta_red, inf.gamma) == (0.43, 32.0, 2.5, 0.47)
    inf = skv.plan_splits([5000, 7000], spec, 8).info()
    assert inf.rho > 0 and inf.delta_attn >= 0


SPEC = skv.AttnSpec(num_q_heads=8, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16)


def _status(fn, *args):
    return fn(*args)


def _plan_call(desc, seq, q=None, num_cu=4, n_ext=0, params=None, ref=None):
    L, Lp = skv._i32(seq)
    qp = None
    if q is not None:
        qa, qp = skv._i32(q)
    h = ctypes.c_void_p()
    refp = None
    if ref is not None:
        ra, refp = skv._i32(ref)
    st = skv._lib.skv_plan_splits(None if desc is None else ctypes.byref(desc), Lp, qp, num_cu, n_ext,
                                  None if params is None else ctypes.byref(params), refp, ctypes.byref(h))
    if st == 0:
        skv._lib.skv_plan_destroy(h)
    return st


def test_plan_argument_errors():
    d = SPEC.desc(2, max_pages=8, num_pages=16)
    assert _plan_call(d, [100, 50]) == 0
    assert _plan_call(None, [100, 50]) == -1
    bad = SPEC.desc(2, max_pages=8, num_pages=16)
    bad.page_size = 8
    assert _plan_call(bad, [100, 50]) == -2
    assert "page_size" in skv._lib.skv_last_error().decode()
    bad = SPEC.desc(2, max_pages=8, num_pages=16)
    bad.num_q_heads = 7
    assert _plan_call(bad, [100, 50]) == -1
    bad = SPEC.desc(2, max_pages=8, num_pages=16)
    bad.head_dim_qk = bad.head_dim_v = 96
    assert _plan_call(bad, [100, 50]) == -2
    assert _plan_call(d, [100, 200]) == -1                       # needs 13 pages > 8
    assert _plan_call(d, [3, 50], q=[4, 1]) == -1                # L < q_len
    assert _plan_call(d, [100, 50], num_cu=0) == -1
    assert _plan_call(d, [100, 50], ref=[2, 1]) == 0
    assert _plan_call(d, [100, 50], ref=[3, 1]) == -1            # more splits than tiles
    p = skv.default_params()
    p.tile_tokens = 32
    assert _plan_call(d, [100, 50], params=p) == -2
    p = skv.default_params()
    p.max_splits = 65
    assert _plan_call(d, [100, 50], params=p) == -1


def test_unsupported_shapes():
    mla = skv.AttnSpec(num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                       mla=True)
    assert _plan_call(mla.desc(1, max_pages=4, num_pages=4), [200]) == 0
    d = mla.desc(1, max_pages=4, num_pages=4)
    d.dtype = skv.SKV_F32
    assert _plan_call(d, [200]) == -2
    d = mla.desc(1, max_pages=4, num_pages=4)
    d.num_q_heads = 100
    assert _plan_call(d, [200]) == -2
    g32 = skv.AttnSpec(num_q_heads=64, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16)
    assert _plan_call(g32.desc(1, max_pages=4, num_pages=4), [60]) == -2


def test_compute_calls_validate_before_launch():
    # Only invalid calls here: each must fail in host validation, never reach a launch.
    plan = skv.plan_splits([100, 50], SPEC, num_cu=4)
    d = SPEC.desc(2, max_pages=8, num_pages=16, scale=0.1)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    st = skv._lib.skv_decode_attn_partial(ctypes.byref(d), None, fake, fake, fake, fake, plan.handle,
                                          fake, fake, fake, None)
    assert st == -1
    d2 = SPEC.desc(3, max_pages=8, num_pages=16)
    st = skv._lib.skv_decode_attn_partial(ctypes.byref(d2), fake, fake, fake, fake, fake, plan.handle,
                                          fake, fake, fake, None)
    assert st == -5
    d3 = SPEC.desc(2, max_pages=2, num_pages=16)             # plan needs 7 pages for L = 100
    st = skv._lib.skv_decode_attn_partial(ctypes.byref(d3), fake, fake, fake, fake, fake, plan.handle,
                                          fake, fake, fake, None)
    assert st == -5
    st = skv._lib.skv_merge_states(ctypes.byref(d), plan.handle, fake, fake, fake, 2, None, None, fake, 0,
                                   None, None)
    assert st == -1                                          # external states missing
    st = skv._lib.skv_merge_states(ctypes.byref(d), plan.handle, fake, fake, fake, 0, None, None, fake, 7,
                                   None, None)
    assert st == -1                                          # bad output dtype
    mla = skv.AttnSpec(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                       mla=True)
    mp = skv.plan_splits([100], mla, num_cu=4)
    dm = mla.desc(1, max_pages=4, num_pages=4)
    st = skv._lib.skv_decode_attn_partial(ctypes.byref(dm), fake, fake, ctypes.c_void_p(512), fake, fake,
                                          mp.handle, fake, fake, fake, None)
    assert st == -1 and "v_pages" in skv._lib.skv_last_error().decode()


def test_upload_rejects_small_workspace():
    plan = skv.plan_splits([100, 50], SPEC, num_cu=4)
    n = plan.workspace_bytes()
    assert n % 256 == 0 and n >= 256
    st = skv._lib.skv_plan_upload(plan.handle, ctypes.c_void_p(256), n - 1, None)
    assert st == -4


def test_plan_export_shapes():
    plan = skv.plan_fixed_chunks([100, 257], skv.AttnSpec(4, 1, 64, 64, 16, dtype=torch.float32), 64)
    e = plan.export()
    assert e["split_counts"].tolist() == [2, 5]
    assert list(zip(e["split_start"], e["split_end"])) == [(0, 64), (64, 100), (0, 64), (64, 128),
                                                            (128, 192), (192, 256), (256, 257)]
    inf = plan.info()
    assert inf.total_splits == 7 and inf.state_rows == 7 * 4 and inf.total_rows == 8
    assert e["state_row_offset"].tolist() == [0, 8, 28]
    assert inf.num_tasks == 7


def test_build_script_loads_without_the_package():
    # the build step must work on a tree with no library yet: loading the
    # build script (as build() does) must not import the package, whose import
    # loads the library
    code = (
        "import importlib.util, sys; "
        f"spec = importlib.util.spec_from_file_location('b', {os.path.join(ROOT, 'split_kv_partial_amd', 'build.py')!r}); "
        "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m); "
        "assert callable(m.build); "
        "assert 'split_kv_partial_amd' not in sys.modules; print('ok')"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_hbm_probe_argument_errors():
    # checked before any launch (no device memory is touched: these addresses
    # are never dereferenced)
    lib = skv._lib
    out = ctypes.c_void_p(4096)
    for buf, nbytes, blocks in [(None, 1024, 8), (4096 + 8, 1024, 8), (4096, 1000, 8), (4096, 0, 8),
                                (4096, 1024, 0), (4096, 1024, 70000)]:
        st = lib.skv_hbm_read_probe(buf, nbytes, out, blocks, None)
        assert st == -1, (buf, nbytes, blocks, st)
    assert lib.skv_hbm_read_probe(4096, 1024, None, 8, None) == -1


def test_mfma_probe_argument_errors():
    # checked before any launch (no address here is dereferenced)
    lib = skv._lib
    out = ctypes.c_void_p(4096)
    for blocks, waves, mw, iters in [(0, 4, 4, 8), (70000, 4, 4, 8), (8, 0, 0, 8), (8, 9, 9, 8),
                                     (8, 4, 5, 8), (8, 4, -1, 8), (8, 4, 4, -1), (8, 4, 4, (1 << 24) + 1)]:
        st = lib.skv_mfma_probe(None, 0, 0, out, blocks, waves, mw, iters, None)
        assert st == -1, (blocks, waves, mw, iters, st)
    assert lib.skv_mfma_probe(None, 0, 0, None, 8, 4, 4, 8, None) == -1
    # streaming waves need a readable, aligned buffer of whole 16-byte chunks
    for buf, nbytes, passes in [(None, 1024, 1), (4096 + 8, 1024, 1), (4096, 1000, 1), (4096, 0, 1),
                                (4096, 1024, -1), (4096, 1024, 2000)]:
        st = lib.skv_mfma_probe(buf, nbytes, passes, out, 8, 8, 4, 8, None)
        assert st == -1, (buf, nbytes, passes, st)


def test_softmax_scale_must_be_positive_and_finite():
    # the MLA kernel's overflow threshold divides by the scale: zero, -0.0,
    # negative and non-finite scales are refused before any launch, by the
    # planner and by both compute calls
    plan = skv.plan_splits([100, 50], SPEC, num_cu=4)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    mla = skv.AttnSpec(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                       mla=True)
    mp = skv.plan_splits([100], mla, num_cu=4)
    for scale in (0.0, -0.0, -0.125, float("inf"), float("-inf"), float("nan")):
        d = SPEC.desc(2, max_pages=8, num_pages=16, scale=scale)
        assert _plan_call(d, [100, 50]) == -1, scale
        assert "softmax_scale" in skv._lib.skv_last_error().decode()
        st = skv._lib.skv_decode_attn_partial(ctypes.byref(d), fake, fake, fake, fake, fake, plan.handle,
                                              fake, fake, fake, None)
        assert st == -1, scale
        st = skv._lib.skv_merge_states(ctypes.byref(d), plan.handle, fake, fake, fake, 0, None, None,
                                       fake, 0, None, None)
        assert st == -1, scale
        dm = mla.desc(1, max_pages=4, num_pages=4, scale=scale)
        st = skv._lib.skv_decode_attn_partial(ctypes.byref(dm), fake, fake, fake, fake, fake, mp.handle,
                                              fake, fake, fake, None)
        assert st == -1, scale
    d = SPEC.desc(2, max_pages=8, num_pages=16, scale=1e-30)
    assert _plan_call(d, [100, 50]) == 0


def _cpu_operands(spec, seq, n_pages=16):
    """CPU tensors shaped as the Python face expects (host-side checks only:
    every call below must raise before reaching the library)."""
    B = len(seq)
    dt = spec.dtype
    q = torch.zeros(B, spec.num_q_heads, spec.head_dim_qk, dtype=dt)
    if spec.mla:
        k = torch.zeros(n_pages, spec.page_size, spec.head_dim_qk, dtype=dt)
        v = k
    else:
        k = torch.zeros(n_pages, spec.num_kv_heads, spec.head_dim_qk, spec.page_size, dtype=dt)
        v = torch.zeros(n_pages, spec.num_kv_heads, spec.head_dim_v, spec.page_size, dtype=dt)
    pt = torch.zeros(B, 8, dtype=torch.int32)
    sl = torch.tensor(seq, dtype=torch.int32)
    return q, k, v, pt, sl


def test_python_face_checks_buffers_before_any_call():
    plan = skv.plan_splits([100, 50], SPEC, num_cu=4)
    inf = plan.info()
    q, k, v, pt, sl = _cpu_operands(SPEC, [100, 50])
    o = torch.zeros(inf.state_rows, 128)
    lse = torch.zeros(inf.state_rows)
    ok = dict(o_part=o, lse_part=lse)

    def bad(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    bad(skv.decode_attn_partial, q.float(), k, v, pt, sl, plan, 0.1, **ok, match="q must have dtype")
    bad(skv.decode_attn_partial, q[:1], k, v, pt, sl, plan, 0.1, **ok, match="q must have shape")
    bad(skv.decode_attn_partial, q, k[:, :1].contiguous(), v, pt, sl, plan, 0.1, **ok, match="k_pages must hold")
    bad(skv.decode_attn_partial, q, k, v[:15], pt, sl, plan, 0.1, **ok, match="v_pages holds")
    bad(skv.decode_attn_partial, q, k, v, pt.long(), sl, plan, 0.1, **ok, match="page_table must have")
    bad(skv.decode_attn_partial, q, k, v, pt[:, :2], sl, plan, 0.1, **ok, match="page_table must be")
    bad(skv.decode_attn_partial, q, k, v, pt, sl[:1], plan, 0.1, **ok, match="seq_lens must have shape")
    bad(skv.decode_attn_partial, q, k, v, pt, sl, plan, 0.1, o_part=o[:-1], lse_part=lse,
        match="o_part holds")
    bad(skv.decode_attn_partial, q, k, v, pt, sl, plan, 0.1, o_part=o.double(), lse_part=lse,
        match="o_part must have dtype")
    bad(skv.decode_attn_partial, q, k, v, pt, sl, plan, 0.1, o_part=o, lse_part=lse[:-1],
        match="lse_part holds")
    rows = inf.total_rows
    out = torch.zeros(rows, 128)
    bad(skv.merge_states, o, lse, plan, o_out=out.half(), lse_out=torch.zeros(rows),
        match="o_out must have dtype")
    bad(skv.merge_states, o, lse, plan, o_out=out[:-1], lse_out=torch.zeros(rows), match="o_out holds")
    bad(skv.merge_states, o, lse, plan, o_out=out, lse_out=torch.zeros(rows - 1), match="lse_out holds")
    bad(skv.merge_states, o[:-1], lse, plan, o_out=out, lse_out=torch.zeros(rows), match="o_part holds")
    bad(skv.merge_states, o, lse, plan, torch.zeros(2, rows, 128), None, o_out=out,
        lse_out=torch.zeros(rows), match="go together")
    bad(skv.merge_states, o, lse, plan, torch.zeros(2, rows, 128).bfloat16(), torch.zeros(2, rows),
        o_out=out, lse_out=torch.zeros(rows), match="o_ext must have dtype")
    bad(skv.merge_states, o, lse, plan, torch.zeros(2, rows - 1, 128), torch.zeros(2, rows - 1),
        o_out=out, lse_out=torch.zeros(rows), match="o_ext must have shape")
    bad(skv.merge_states, o, lse, plan, torch.zeros(2, rows, 128), torch.zeros(3, rows),
        o_out=out, lse_out=torch.zeros(rows), match="lse_ext must have shape")
    bad(skv.merge_states, o, lse, plan, out_dtype=torch.float16, match="out_dtype")
    # MLA: values are the key rows
    mla = skv.AttnSpec(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                       mla=True)
    mp = skv.plan_splits([100], mla, num_cu=4)
    q, k, v, pt, sl = _cpu_operands(mla, [100], n_pages=4)
    mi = mp.info()
    mo, ml = torch.zeros(mi.state_rows, 512), torch.zeros(mi.state_rows)
    bad(skv.decode_attn_partial, q, k, k.clone(), pt, sl, mp, 0.1, o_part=mo, lse_part=ml,
        match="v_pages must be k_pages")
    bad(skv.decode_attn_partial, q, k[:, :, :512].contiguous(), k[:, :, :512].contiguous(), pt, sl,
        mp, 0.1, o_part=mo, lse_part=ml, match="v_pages must be k_pages")


def test_whole_path_scratch_size_and_checks():
    plan = skv.plan_splits([100, 50], SPEC, num_cu=4)
    inf = plan.info()
    need = skv.scratch_bytes(plan)
    # counters block (128 bytes of merge arguments, then three launch counters
    # and one per request, each on a 256-byte line of its own), then o_part and
    # lse_part, each 256-aligned
    up = lambda x: (x + 255) // 256 * 256
    assert need == up(128 + 256 * (3 + 2)) + up(inf.state_rows * 128 * 4) + up(inf.state_rows * 4)
    assert skv._lib.skv_decode_attn_scratch_bytes(None) == 0
    d = SPEC.desc(2, max_pages=8, num_pages=16, scale=0.1)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    call = lambda scratch, nbytes, n_ext=0, ext=None: skv._lib.skv_decode_attn(
        ctypes.byref(d), fake, fake, fake, fake, fake, plan.handle, fake, scratch, nbytes, n_ext, ext,
        ext, fake, 0, None, None)
    assert call(fake, need - 1) == -4 and "scratch" in skv._lib.skv_last_error().decode()
    assert call(None, need) == -1
    assert call(fake, need, n_ext=2) == -1                       # external states missing
    st = skv._lib.skv_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, plan.handle, fake, fake,
                                  need, 0, None, None, fake, 5, None, None)
    assert st == -1                                              # bad output dtype
    d.softmax_scale = 0.0
    assert call(fake, need) == -1


def test_query_tile_defaults_and_limits():
    # tokens per attention task: the bf16 matrix-core GQA kernel fills 128
    # rows of (token, head); every other kernel takes one token per task
    cases = [(torch.bfloat16, 32, 2, 128, False, 8), (torch.bfloat16, 32, 2, 64, False, 8),
             (torch.bfloat16, 16, 2, 128, False, 16), (torch.bfloat16, 16, 2, 64, False, 16),
             (torch.bfloat16, 8, 2, 128, False, 1), (torch.float32, 32, 2, 128, False, 1),
             (torch.bfloat16, 128, 1, 576, True, 1)]
    seq, q = [300, 90], [20, 1]
    for dt, hq, hkv, d, mla, qt in cases:
        spec = skv.AttnSpec(hq, hkv, d, 512 if mla else d, 16, dtype=dt, mla=mla)
        plan = skv.plan_splits(seq, spec, 64, q_lens=q)
        assert plan.info().query_tile == qt, (dt, hq, hkv, d)
        # one task per (request, KV head, query tile, split)
        counts = plan.export()["split_counts"]
        assert plan.info().num_tasks == sum(int(c) * hkv * -(-n // qt) for c, n in zip(counts, q))
    spec = skv.AttnSpec(32, 2, 128, 128, 16, dtype=torch.bfloat16)
    prm = skv.default_params()
    for qt in (1, 2, 8):
        prm.query_tile = qt
        assert skv.plan_splits(seq, spec, 64, q_lens=q, params=prm).info().query_tile == qt
    prm.query_tile = 9          # 9 tokens x 16 heads = 144 rows: more than the kernel's 128
    with pytest.raises(skv.SplitKVError):
        skv.plan_splits(seq, spec, 64, q_lens=q, params=prm)
    prm.query_tile = 2          # the one-token kernels take only tiles of one
    with pytest.raises(skv.SplitKVError):
        skv.plan_splits(seq, skv.AttnSpec(8, 2, 128, 128, 16, dtype=torch.float32), 64, q_lens=q,
                        params=prm)


def test_fp8_descriptions_and_entry_point_checks():
    f8 = skv.AttnSpec(num_q_heads=32, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                      dtype=skv.FP8)
    assert _plan_call(f8.desc(1, max_pages=8, num_pages=8), [100]) == 0
    for hq, hkv, d in ((8, 2, 128), (4, 4, 64), (64, 2, 128)):      # groups of 4, 1, 32
        g = skv.AttnSpec(hq, hkv, d, d, 16, dtype=skv.FP8)
        assert _plan_call(g.desc(1, max_pages=8, num_pages=8), [100]) == -2
    # FP8 MLA rows: planned like bf16 rows; one scale per page, so the value
    # scales must be the key scales (checked before any launch)
    mla = skv.AttnSpec(128, 1, 576, 512, 64, dtype=skv.FP8, mla=True)
    assert _plan_call(mla.desc(1, max_pages=4, num_pages=4), [100]) == 0
    mplan = skv.plan_splits([100, 300], mla, num_cu=4)
    md = mla.desc(2, max_pages=8, num_pages=16, scale=0.1)
    fk = ctypes.c_void_p(256)
    mcall = lambda ks, vs, vp: skv._lib.skv_decode_attn_partial_fp8(
        ctypes.byref(md), fk, fk, vp, ks, vs, fk, fk, mplan.handle, fk, fk, fk, None)
    assert mcall(fk, ctypes.c_void_p(512), fk) == -1 and "v_scales" in skv._lib.skv_last_error().decode()
    assert mcall(fk, fk, ctypes.c_void_p(512)) == -1 and "v_pages" in skv._lib.skv_last_error().decode()
    bad = f8.desc(1, max_pages=8, num_pages=8)
    bad.dtype = 3
    assert _plan_call(bad, [100]) == -1
    # FP8 plans run one query token per task
    prm = skv.default_params()
    prm.query_tile = 2
    with pytest.raises(skv.SplitKVError):
        skv.plan_splits([100], f8, 64, q_lens=[5], params=prm)
    plan = skv.plan_splits([100, 50], f8, num_cu=4, q_lens=[3, 1])
    assert plan.info().query_tile == 1
    d = f8.desc(2, max_pages=8, num_pages=16, scale=0.1)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    call = lambda desc, ks, vs: skv._lib.skv_decode_attn_partial_fp8(
        ctypes.byref(desc), fake, fake, fake, ks, vs, fake, fake, plan.handle, fake, fake, fake, None)
    assert call(d, None, fake) == -1 and "scales" in skv._lib.skv_last_error().decode()
    assert call(d, fake, None) == -1
    bf = SPEC.desc(2, max_pages=8, num_pages=16, scale=0.1)     # a bf16 description
    assert call(bf, fake, fake) == -1
    # the bf16 entry points refuse FP8 descriptions (no scales to pass)
    st = skv._lib.skv_decode_attn_partial(ctypes.byref(d), fake, fake, fake, fake, fake, plan.handle, fake,
                                          fake, fake, None)
    assert st == -1 and "scales" in skv._lib.skv_last_error().decode()
    need = skv.scratch_bytes(plan)
    st = skv._lib.skv_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, plan.handle, fake, fake, need,
                                  0, None, None, fake, 0, None, None)
    assert st == -1
    # the FP8 one-call entry point: an FP8 description, its scales, and a plan
    # for the two launches (the one-launch engine has no FP8 kernels)
    fcall = lambda desc, ks, vs, pl: skv._lib.skv_decode_attn_fp8(
        ctypes.byref(desc), fake, fake, fake, ks, vs, fake, fake, pl.handle, fake, fake,
        skv.scratch_bytes(pl), 0, None, None, fake, 0, None, None)
    assert fcall(bf, fake, fake, plan) == -1 and "SKV_FP8_E4M3" in skv._lib.skv_last_error().decode()
    assert fcall(d, None, fake, plan) == -1 and "scales" in skv._lib.skv_last_error().decode()
    prm1 = skv.default_params()
    prm1.overlap_reduction = 1
    plan1 = skv.plan_splits([100, 50], f8, num_cu=4, q_lens=[3, 1], params=prm1)
    assert fcall(d, fake, fake, plan1) == -2 and "overlap_reduction" in skv._lib.skv_last_error().decode()
    # the Python face: FP8 specs go through decode_attn_partial_fp8 only
    with pytest.raises(ValueError):
        skv.decode_attn_partial(torch.empty(0), None, None, None, None, plan, 0.1)


def test_library_defaults_are_the_calibration_tools_fit():
    # the table the library compiles in is the one the calibration tool wrote
    # beside profiles/mi355x.json: every kernel's default parameters equal it
    import json
    fit = json.load(open(os.path.join(ROOT, "profiles", "mi355x.json")))["kernels"]
    specs = {"gqa_mfma": skv.AttnSpec(128, 8, 128, 128, 16),
             "gqa_mfma_g8": skv.AttnSpec(64, 8, 128, 128, 16),
             "gqa_valu": skv.AttnSpec(32, 8, 128, 128, 16, dtype=torch.float32),
             "mla_mfma": skv.AttnSpec(128, 1, 576, 512, 64, mla=True)}
    for kernel, spec in specs.items():
        inf = skv.plan_splits([5000, 7000], spec, 64).info()
        c = fit[kernel]
        assert (inf.rho, inf.delta_attn, inf.delta_red, inf.gamma) == (c["rho"], c["delta_attn"], c["delta_red"],
                                                                      c["gamma"]), kernel
        assert inf.tile_time_us == c["tile_time_us"] and inf.balanced_candidates == c["balanced"], kernel
        assert c["rmse_attn_us"] > 0 and len(c["points"]) >= 10
