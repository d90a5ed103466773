"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from draft_attention_token_amd import specprefill as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specprefill.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sp_status|int|const char \*|size_t)\s*\*?\s*(sp_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_expected_functions():
    assert _declared() == sorted(sp.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = sp.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.sp_abi_version() == 3


def test_status_strings():
    assert sp.status_string(0) == "ok"
    assert "invalid" in sp.status_string(1)
    assert "unsupported" in sp.status_string(2)
    assert "workspace" in sp.status_string(3)
    assert sp.status_string(99) == "unknown status"


def _score(desc, batch, q=1, k=1, out=1, ws=1, ws_bytes=1 << 30):
    # Non-null fake pointers: validation must reject before touching them.
    vp = lambda v: ctypes.c_void_p(v * 4096 if v else 0)
    return sp.lib().sp_score_attention(ctypes.byref(desc), batch.ref() if batch else None,
                                       vp(q), vp(k), vp(out), vp(ws), ws_bytes, None)


def _desc(**kw):
    base = dict(n_layers=6, n_q_heads=16, n_kv_heads=4, head_dim=128, n_lookahead=8,
                dtype=torch.bfloat16, scale=None, algo="two_pass")
    base.update(kw)
    return sp.attn_desc(**base)


@pytest.mark.parametrize("kw, want", [
    (dict(n_layers=0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(n_q_heads=0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(n_kv_heads=3), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(n_lookahead=0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(dtype=torch.float16), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(algo=7), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), sp.SP_ERR_UNSUPPORTED),
    (dict(n_lookahead=9), sp.SP_ERR_UNSUPPORTED),           # L * G = 36 > 32
    (dict(n_q_heads=64, n_kv_heads=4), sp.SP_ERR_UNSUPPORTED),
    (dict(n_lookahead=-1), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(prefill_row=2), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(n_lookahead=8, prefill_row=True), sp.SP_ERR_UNSUPPORTED),   # (8 + 1) * 4 > 32
    (dict(row_pool=-1), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(row_pool=12), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(row_pool=35), sp.SP_ERR_UNSUPPORTED),
    (dict(row_pool=13, algo="stream"), sp.SP_ERR_UNSUPPORTED),
    (dict(row_pool=13, dtype=torch.bfloat16, k_dtype=torch.float8_e4m3fn, k_scales=[0.01] * 24),
     sp.SP_ERR_UNSUPPORTED),
])
def test_score_rejects_bad_descriptors(kw, want):
    assert _score(_desc(**kw), sp.Batch([0, 100])) == want


def _fp8(**kw):
    base = dict(dtype=torch.bfloat16, k_dtype=torch.float8_e4m3fn, algo="auto",
                k_scales=[0.01] * 24)
    base.update(kw)
    return _desc(**base)


@pytest.mark.parametrize("kw, want", [
    (dict(k_scales=None), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(k_scales=[0.01] * 23 + [0.0]), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(k_scales=[0.01] * 23 + [-1.0]), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(k_scales=[float("inf")] + [0.01] * 23), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(k_scales=[float("nan")] * 24), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(algo="two_pass"), sp.SP_ERR_UNSUPPORTED),           # fp8 K: single-pass kernel only
    (dict(n_layers=40, n_kv_heads=4, k_scales=[0.01] * 160), sp.SP_ERR_UNSUPPORTED),  # > 128
])
def test_score_rejects_bad_fp8_key_scales(kw, want):
    assert _score(_fp8(**kw), sp.Batch([0, 100])) == want


def test_fp8_descriptor_fields():
    d = _fp8()
    assert d.dtype == sp.SP_DTYPE_BF16_FP8K
    assert [d.k_scales[i] for i in range(24)] == pytest.approx([0.01] * 24)
    # fp8 Q, or fp8 K under fp32 Q, has no code
    assert _desc(dtype=torch.float32, k_dtype=torch.float8_e4m3fn).dtype == -1
    assert _desc(dtype=torch.float8_e4m3fn).dtype == -1


@pytest.mark.parametrize("offsets, want", [
    ([5, 10], sp.SP_ERR_INVALID_ARGUMENT),          # does not start at 0
    ([0, 10, 10], sp.SP_ERR_INVALID_ARGUMENT),      # empty prompt
    ([0, 10, 7], sp.SP_ERR_INVALID_ARGUMENT),       # decreasing
    ([0], sp.SP_ERR_INVALID_ARGUMENT),              # no prompts
    (list(range(0, 130)), sp.SP_ERR_UNSUPPORTED),    # 129 prompts > SP_MAX_PROMPTS
    ([0, 1 << 30], sp.SP_ERR_UNSUPPORTED),           # too many tokens
])
def test_score_rejects_bad_batches(offsets, want):
    assert _score(_desc(), sp.Batch(offsets)) == want


def test_score_rejects_null_and_misaligned_pointers_and_small_workspace():
    b = sp.Batch([0, 100])
    assert _score(_desc(), None) == sp.SP_ERR_INVALID_ARGUMENT
    assert _score(_desc(), b, q=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _score(_desc(), b, k=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _score(_desc(), b, out=0) == sp.SP_ERR_INVALID_ARGUMENT
    L = sp.lib()
    d = _desc()
    assert L.sp_score_attention(ctypes.byref(d), b.ref(), ctypes.c_void_p(4100),
                                ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                                ctypes.c_void_p(4096), 1 << 30, None) == sp.SP_ERR_INVALID_ARGUMENT
    need = sp.score_workspace_bytes(d, b)
    assert need > 0
    assert _score(d, b, ws_bytes=need - 1) == sp.SP_ERR_WORKSPACE_TOO_SMALL
    assert _score(d, b, ws=0) == sp.SP_ERR_WORKSPACE_TOO_SMALL


def test_workspace_sizes_grow_with_the_batch():
    d = _desc()
    small = sp.score_workspace_bytes(d, sp.Batch([0, 1000]))
    big = sp.score_workspace_bytes(d, sp.Batch([0, 100000]))
    assert 0 < small < big
    pd = sp.pool_desc()
    # per-block (min, max) of 1024-token blocks, and one per prompt
    assert sp.pool_workspace_bytes(pd, sp.Batch([0, 5000])) >= 5 * 8 + 8
    assert sp.pool_workspace_bytes(pd, sp.Batch([0, 5000])) < \
        sp.pool_workspace_bytes(pd, sp.Batch([0, 5000000]))
    assert sp.select_workspace_bytes(sp.Batch([0, 5000]), 32) == 0   # selection needs none
    assert sp.gather_workspace_bytes(sp.Batch([0, 5000]), 32) >= 157 * 4


def _pool(desc, batch, imp=1, cs=1, ws=1, ws_bytes=1 << 30):
    vp = lambda v: ctypes.c_void_p(v * 4096 if v else 0)
    return sp.lib().sp_pool_chunk(ctypes.byref(desc), batch.ref(), vp(imp), None, vp(cs), vp(ws),
                                  ws_bytes, None)


@pytest.mark.parametrize("kw, want", [
    (dict(W=12), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(W=0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(W=131), sp.SP_ERR_UNSUPPORTED),
    (dict(C=0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(C=2048), sp.SP_ERR_UNSUPPORTED),
    (dict(first_n=-1), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(first_mult=0.0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(last_mult=float("inf")), sp.SP_ERR_INVALID_ARGUMENT),
])
def test_pool_rejects_bad_descriptors(kw, want):
    assert _pool(sp.pool_desc(**kw), sp.Batch([0, 100])) == want


def test_pool_rejects_null_outputs_and_small_workspace():
    b = sp.Batch([0, 100])
    assert _pool(sp.pool_desc(), b, imp=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _pool(sp.pool_desc(), b, cs=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _pool(sp.pool_desc(), b, ws_bytes=8) == sp.SP_ERR_WORKSPACE_TOO_SMALL


def _select(mode, param, batch, C=32, cs=1, keep=1, cnt=1):
    vp = lambda v: ctypes.c_void_p(v * 4096 if v else 0)
    return sp.lib().sp_select_chunks(mode, param, batch.ref(), C, vp(cs), vp(keep), vp(cnt), None,
                                     0, None)


@pytest.mark.parametrize("mode, param, C, want", [
    (5, 0.5, 32, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_TOP_P, 0.0, 32, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_TOP_P, 1.01, 32, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_MASS, -0.5, 32, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_MASS, float("nan"), 32, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_MASS, 0.85, 0, sp.SP_ERR_INVALID_ARGUMENT),
    (sp.SP_SELECT_MASS, 0.85, 1, sp.SP_ERR_UNSUPPORTED),     # 100000 chunks > 16384
])
def test_select_rejects_bad_arguments(mode, param, C, want):
    assert _select(mode, param, sp.Batch([0, 100000]), C) == want


def test_select_and_gather_reject_null_pointers():
    b = sp.Batch([0, 100])
    assert _select(sp.SP_SELECT_MASS, 0.85, b, cs=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _select(sp.SP_SELECT_MASS, 0.85, b, keep=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert _select(sp.SP_SELECT_MASS, 0.85, b, cnt=0) == sp.SP_ERR_INVALID_ARGUMENT
    vp = lambda v: ctypes.c_void_p(v)
    L = sp.lib()
    args = [vp(4096)] * 5
    assert L.sp_gather_kept(b.ref(), 32, vp(0), *args[:4], vp(4096), 1 << 20, None) == \
        sp.SP_ERR_INVALID_ARGUMENT
    assert L.sp_gather_kept(b.ref(), 32, *args, vp(4096), 4, None) == sp.SP_ERR_WORKSPACE_TOO_SMALL
    assert L.sp_gather_kept(b.ref(), 0, *args, vp(4096), 1 << 20, None) == sp.SP_ERR_INVALID_ARGUMENT


def _post(batch, desc=None, mode=sp.SP_SELECT_MASS, param=0.85, null=(), ws_bytes=1 << 30,
          ws=4096):
    """sp_pool_select_gather with fake (never dereferenced) device pointers;
    the arguments named in `null` are passed as NULL."""
    names = ["importance", "token_ids", "token_scores", "chunk_scores", "keep", "n_kept",
             "kept_ids", "kept_pos", "kept_offsets"]
    ptrs = [ctypes.c_void_p(0 if n in null else 4096 * (i + 1)) for i, n in enumerate(names)]
    d = desc if desc is not None else sp.pool_desc()
    return sp.lib().sp_pool_select_gather(ctypes.byref(d), mode, param, batch.ref(), *ptrs,
                                          ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw, want", [
    (dict(mode=7), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(param=0.0), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(param=float("nan")), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(mode=sp.SP_SELECT_TOP_P, param=1.5), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(desc=sp.pool_desc(W=4)), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(desc=sp.pool_desc(C=0)), sp.SP_ERR_INVALID_ARGUMENT),
    (dict(desc=sp.pool_desc(C=2048)), sp.SP_ERR_UNSUPPORTED),
    (dict(desc=sp.pool_desc(C=1)), sp.SP_ERR_UNSUPPORTED),      # 100000 chunks in a prompt
    (dict(ws=4100), sp.SP_ERR_INVALID_ARGUMENT),                  # misaligned workspace
    (dict(ws_bytes=64), sp.SP_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=0), sp.SP_ERR_WORKSPACE_TOO_SMALL),
])
def test_pool_select_gather_rejects_bad_arguments(kw, want):
    assert _post(sp.Batch([0, 100000]), **kw) == want


@pytest.mark.parametrize("name", ["importance", "token_ids", "chunk_scores", "keep", "n_kept",
                                  "kept_ids", "kept_pos", "kept_offsets"])
def test_pool_select_gather_rejects_null_pointers(name):
    assert _post(sp.Batch([0, 100]), null=(name,)) == sp.SP_ERR_INVALID_ARGUMENT


def test_pool_select_gather_workspace_covers_every_form():
    pd = sp.pool_desc()
    for offs in ([0, 100], [0, 5000, 5001], [0, 131072], [0] + [4096 * (i + 1) for i in range(64)]):
        b = sp.Batch(offs)
        nc = b.n_chunks(32)
        need = sp.post_workspace_bytes(pd, b)
        # status header + two 8-byte slots per pool group (256 tokens at C = 32),
        # one per block (up to 1024) and one per chunk
        groups = sum((n + 255) // 256 for n in np.diff(offs))
        assert need >= 256 + groups * 16 + 1024 * 8 + nc * 8
        # the die-local form: per die two copies of a slot per group min, max,
        # chunk and prompt
        assert need >= 256 + 2 * 8 * (2 * groups + nc + len(offs) - 1) * 8
        # or the separate kernels' own workspaces
        assert need >= 256 + sp.pool_workspace_bytes(pd, b) + sp.gather_workspace_bytes(b, 32)
    # form queries are host arithmetic (no device here: the separate kernels)
    assert sp.post_plan(pd, sp.Batch([0, 131072])) in (0, 512, 4096)
    assert sp.post_form(pd, sp.Batch([0, 131072])) in (("separate", 0), ("die", 4096))


def test_pool_select_gather_form_rejects_bad_arguments():
    L = sp.lib()
    b = sp.Batch([0, 1000])
    f, tb = ctypes.c_int32(0), ctypes.c_int32(0)
    pd = sp.pool_desc()
    assert L.sp_pool_select_gather_form(ctypes.byref(pd), b.ref(), None, ctypes.byref(tb)) == \
        sp.SP_ERR_INVALID_ARGUMENT
    assert L.sp_pool_select_gather_form(ctypes.byref(pd), b.ref(), ctypes.byref(f), None) == \
        sp.SP_ERR_INVALID_ARGUMENT
    bad = sp.pool_desc(W=4)
    assert L.sp_pool_select_gather_form(ctypes.byref(bad), b.ref(), ctypes.byref(f),
                                        ctypes.byref(tb)) == sp.SP_ERR_INVALID_ARGUMENT
    assert L.sp_pool_select_gather_form(ctypes.byref(pd), None, ctypes.byref(f),
                                        ctypes.byref(tb)) == sp.SP_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sp, "_lib", None)
    monkeypatch.setattr(sp, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not found"):
        sp.lib()


def test_break_even_matches_oracle_and_defaults():
    import oracle
    for n in (1, 600, 5400, 100000):
        for f in (0.0, 0.3, 0.45, 0.46, 0.47, 0.9, 1.0):
            kept = int(round(f * n))
            assert sp.break_even(n, kept) == oracle.break_even(n, kept), (n, kept)
            assert sp.break_even(n, kept, 995.0, 270.0, 1.5) == \
                oracle.break_even(n, kept, 995.0, 270.0, 1.5), (n, kept)


@pytest.mark.parametrize("args", [
    (0, 0, 0, 0, 0), (10, 11, 0, 0, 0), (10, -1, 0, 0, 0), (10, 5, float("nan"), 0, 0),
    (10, 5, 0, float("inf"), 0),
])
def test_break_even_rejects_bad_arguments(args):
    run = ctypes.c_int32()
    assert sp.lib().sp_break_even(*args, ctypes.byref(run)) == sp.SP_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("n, W, s", [(4471, 2000, 1000), (1, 2000, 1000), (2000, 2000, 1000),
                                     (2001, 2000, 1000), (131072, 8192, 4096), (5000, 1000, 300),
                                     (777, 100, 100)])
def test_window_plan_matches_oracle(n, W, s):
    import oracle
    starts, lengths, keeps = sp.window_plan(n, W, s)
    assert list(zip(starts, lengths, keeps)) == oracle.window_plan(n, W, s)


def test_window_plan_rejects_bad_arguments_and_reports_size():
    L = sp.lib()
    n = ctypes.c_int32()
    for args in [(0, 10, 5), (10, 0, 1), (10, 5, 6), (10, 5, 0)]:
        assert L.sp_window_plan(*args, 0, None, None, None, ctypes.byref(n)) == \
            sp.SP_ERR_INVALID_ARGUMENT
    st, ln, kp = (ctypes.c_int64 * 2)(), (ctypes.c_int32 * 2)(), (ctypes.c_int32 * 2)()
    assert L.sp_window_plan(4471, 2000, 1000, 2, st, ln, kp, ctypes.byref(n)) == \
        sp.SP_ERR_INVALID_ARGUMENT
    assert n.value == 4                                   # the capacity it needs
    assert L.sp_window_plan(4471, 2000, 1000, 4, None, None, None, ctypes.byref(n)) == \
        sp.SP_ERR_INVALID_ARGUMENT


def test_stitch_and_legacy_reject_bad_arguments():
    L = sp.lib()
    vp = lambda v: ctypes.c_void_p(v)
    win = sp.Batch([0, 2000, 4000])
    st = (ctypes.c_int64 * 2)(0, 1000)
    kp = (ctypes.c_int32 * 2)(1000, 2000)
    assert L.sp_stitch_windows(win.ref(), st, kp, 3000, vp(4096), vp(0), None) == \
        sp.SP_ERR_INVALID_ARGUMENT                        # null output
    assert L.sp_stitch_windows(win.ref(), st, kp, 2999, vp(4096), vp(4096), None) == \
        sp.SP_ERR_INVALID_ARGUMENT                        # keep range past the prompt
    kp2 = (ctypes.c_int32 * 2)(1000, 2001)
    assert L.sp_stitch_windows(win.ref(), st, kp2, 4000, vp(4096), vp(4096), None) == \
        sp.SP_ERR_INVALID_ARGUMENT                        # keeps more than the window holds
    b = sp.Batch([0, 500])
    args = [vp(4096)] * 5
    ok = dict(C=32, keep=0.3, mn=128, mx=2000)
    def call(C=32, keep=0.3, mn=128, mx=2000, ws_bytes=1 << 20):
        return L.sp_select_legacy(b.ref(), C, keep, mn, mx, *args, vp(4096), ws_bytes, None)
    assert call(keep=0.0) == sp.SP_ERR_INVALID_ARGUMENT
    assert call(keep=float("nan")) == sp.SP_ERR_INVALID_ARGUMENT
    assert call(mn=-1) == sp.SP_ERR_INVALID_ARGUMENT
    assert call(mx=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert call(C=0) == sp.SP_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=4) == sp.SP_ERR_WORKSPACE_TOO_SMALL
    assert sp.select_legacy_workspace_bytes(b, 32) >= 16 + 4


def test_bench_read_aids_load_and_refuse_bad_shapes():
    """bench.py's measurement aids (libspbench.so, outside the product
    library) load and export the plain read and the K-order read; the K-order
    read refuses a segment that is not whole 16-byte chunks, or whose chunk
    count does not divide the block, before launching anything."""
    lib = ctypes.CDLL(os.path.join(ROOT, "draft_attention_token_amd", "libspbench.so"))
    assert hasattr(lib, "spbench_read") and hasattr(lib, "spbench_read_heads")
    fn = lib.spbench_read_heads
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    for seg in (24, 16 * 3, 0):        # not whole chunks; 3 chunks do not divide 512; none
        assert fn(None, 6, 1000, 4, seg, None, 248, None) != 0, seg
    assert fn(None, 0, 1000, 4, 256, None, 248, None) != 0   # no layer
    assert fn(None, 6, 1000, 4, 256, None, 0, None) != 0     # no block
