"""Python binding of libspecprefill (ctypes; argument marshalling only).

Every step of the path runs in the library's HIP kernels. torch is used for
device memory and the current HIP stream. Importing this module does not need
a GPU; calling a function does. If the shared library is missing, every call
raises: there is no fallback path.

Functions mirror the C ABI in ``include/specprefill.h``:

* :func:`sp_score_attention` (Q, K -> importance)
* :func:`sp_pool_chunk` (importance -> token scores, chunk scores)
* :func:`sp_select_chunks` (chunk scores -> keep flags, kept-chunk counts)
* :func:`sp_gather_kept` (keep flags, token ids -> kept ids, positions, offsets)
* :func:`sp_pool_select_gather` (the three calls above as one)

``offsets`` is always the host-side ``[B + 1]`` int64 prompt-token offsets.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SP_LIB_PATH names another build of the library (the host-sanitizer checks
# load one); by default the in-tree build.
LIB_PATH = os.environ.get("SP_LIB_PATH") or os.path.join(_HERE, "libspecprefill.so")

SP_OK, SP_ERR_INVALID_ARGUMENT, SP_ERR_UNSUPPORTED, SP_ERR_WORKSPACE_TOO_SMALL, SP_ERR_DEVICE = range(5)
SP_DTYPE_F32, SP_DTYPE_BF16, SP_DTYPE_BF16_FP8K = 0, 1, 2
SP_SELECT_TOP_P, SP_SELECT_MASS = 0, 1
SP_SCORE_AUTO, SP_SCORE_TWO_PASS, SP_SCORE_STREAM = 0, 1, 2
SP_MAX_PROMPTS = 128

EXPORTED = [
    "sp_abi_version", "sp_status_string", "sp_score_workspace_bytes", "sp_pool_workspace_bytes",
    "sp_select_workspace_bytes", "sp_gather_workspace_bytes", "sp_score_attention",
    "sp_pool_chunk", "sp_select_chunks", "sp_gather_kept", "sp_score_status", "sp_break_even",
    "sp_window_plan", "sp_stitch_windows", "sp_select_legacy_workspace_bytes", "sp_select_legacy",
    "sp_score_plan", "sp_score_attention_noalloc", "sp_pool_select_gather_workspace_bytes",
    "sp_pool_select_gather", "sp_pool_select_gather_plan", "sp_pool_select_gather_form",
]

_ALGOS = {"auto": SP_SCORE_AUTO, "two_pass": SP_SCORE_TWO_PASS, "stream": SP_SCORE_STREAM}
_MODES = {"top_p": SP_SELECT_TOP_P, "mass": SP_SELECT_MASS}


class SpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class sp_batch(ctypes.Structure):
    _fields_ = [("n_prompts", ctypes.c_int32), ("token_offsets", ctypes.POINTER(ctypes.c_int64))]


class sp_attn_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_lookahead", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("algo", ctypes.c_int32),
                ("k_scales", ctypes.POINTER(ctypes.c_float)), ("prefill_row", ctypes.c_int32),
                ("row_pool", ctypes.c_int32)]


class sp_pool_desc(ctypes.Structure):
    _fields_ = [("pool_window", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("normalize", ctypes.c_int32), ("boost_first_n", ctypes.c_int32),
                ("boost_first_mult", ctypes.c_float), ("boost_last_n", ctypes.c_int32),
                ("boost_last_mult", ctypes.c_float)]


_lib = None


def lib():
    """The loaded shared library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libspecprefill.so not found at {LIB_PATH}; build it with "
                               "`python -m draft_attention_token_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, szp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
        bp = ctypes.POINTER(sp_batch)
        L.sp_abi_version.restype = ctypes.c_int
        L.sp_status_string.argtypes = [ctypes.c_int]
        L.sp_status_string.restype = ctypes.c_char_p
        L.sp_score_workspace_bytes.argtypes = [ctypes.POINTER(sp_attn_desc), bp, szp]
        L.sp_pool_workspace_bytes.argtypes = [ctypes.POINTER(sp_pool_desc), bp, szp]
        L.sp_select_workspace_bytes.argtypes = [bp, ctypes.c_int32, szp]
        L.sp_gather_workspace_bytes.argtypes = [bp, ctypes.c_int32, szp]
        L.sp_score_attention.argtypes = [ctypes.POINTER(sp_attn_desc), bp, vp, vp, vp, vp, sz, vp]
        L.sp_pool_chunk.argtypes = [ctypes.POINTER(sp_pool_desc), bp, vp, vp, vp, vp, sz, vp]
        L.sp_select_chunks.argtypes = [ctypes.c_int32, ctypes.c_double, bp, ctypes.c_int32, vp, vp,
                                       vp, vp, sz, vp]
        L.sp_gather_kept.argtypes = [bp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sp_score_status.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
        L.sp_score_attention_noalloc.argtypes = [ctypes.POINTER(sp_attn_desc), bp, vp, vp, vp, vp]
        L.sp_score_plan.argtypes = [ctypes.POINTER(sp_attn_desc), bp, ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.sp_pool_select_gather_workspace_bytes.argtypes = [ctypes.POINTER(sp_pool_desc), bp, szp]
        L.sp_pool_select_gather.argtypes = [ctypes.POINTER(sp_pool_desc), ctypes.c_int32,
                                            ctypes.c_double, bp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
        L.sp_pool_select_gather_plan.argtypes = [ctypes.POINTER(sp_pool_desc), bp,
                                                 ctypes.POINTER(ctypes.c_int32)]
        L.sp_break_even.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]
        i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        L.sp_window_plan.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     i64p, i32p, i32p, i32p]
        L.sp_stitch_windows.argtypes = [bp, i64p, i32p, ctypes.c_int64, vp, vp, vp]
        L.sp_select_legacy_workspace_bytes.argtypes = [bp, ctypes.c_int32, szp]
        L.sp_select_legacy.argtypes = [bp, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                       ctypes.c_int32, vp, vp, vp, vp, vp, vp, sz, vp]
        for name in EXPORTED[2:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sp_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SP_OK:
        raise SpError(status, where)


class Batch:
    """Host-side batch descriptor; keeps the offsets array alive."""

    def __init__(self, offsets):
        if isinstance(offsets, torch.Tensor):
            offsets = offsets.detach().cpu().numpy()
        self.offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        self.struct = sp_batch(len(self.offsets) - 1,
                               self.offsets.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))

    @property
    def B(self) -> int:
        return len(self.offsets) - 1

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    def n_chunks(self, C: int) -> int:
        return int(sum((int(self.offsets[b + 1] - self.offsets[b]) + C - 1) // C for b in range(self.B)))

    def ref(self):
        return ctypes.byref(self.struct)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    # Zero-filled: the scoring workspace must start out zeroed (calls leave it
    # ready for the next call); the others do not care.
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def attn_desc(n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, dtype, scale=None,
              algo="auto", k_dtype=None, k_scales=None, prefill_row=False,
              row_pool=1) -> sp_attn_desc:
    """dtype: Q's torch dtype (and K's unless k_dtype says otherwise).
    k_dtype=torch.float8_e4m3fn with bf16 Q selects fp8 K codes; k_scales
    is then the [n_layers * n_kv_heads] fp32 host array of key scales.
    prefill_row: Q carries one more step in front, the prompt's last row.
    row_pool: odd W > 1 pools every probability row before the max."""
    if k_dtype is None or k_dtype == dtype:
        dt = {torch.float32: SP_DTYPE_F32, torch.bfloat16: SP_DTYPE_BF16}.get(dtype, -1)
    elif dtype == torch.bfloat16 and k_dtype == torch.float8_e4m3fn:
        dt = SP_DTYPE_BF16_FP8K
    else:
        dt = -1
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    desc = sp_attn_desc(n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, dt, float(scale),
                        _ALGOS[algo] if isinstance(algo, str) else int(algo), None,
                        int(prefill_row) if isinstance(prefill_row, (bool, int)) else -1,
                        int(row_pool))
    if k_scales is not None:
        ks = np.ascontiguousarray(np.asarray(
            k_scales.cpu() if isinstance(k_scales, torch.Tensor) else k_scales,
            dtype=np.float32).reshape(-1))
        desc._k_scales = ks   # the descriptor points into it: keep it alive with the descriptor
        desc.k_scales = ks.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    return desc


def pool_desc(W=13, C=32, normalize=True, first_n=64, first_mult=1.5, last_n=128,
              last_mult=1.3) -> sp_pool_desc:
    return sp_pool_desc(W, C, int(bool(normalize)), first_n, first_mult, last_n, last_mult)


def score_workspace_bytes(desc: sp_attn_desc, batch: Batch) -> int:
    n = ctypes.c_size_t()
    _check(lib().sp_score_workspace_bytes(ctypes.byref(desc), batch.ref(), ctypes.byref(n)),
           "sp_score_workspace_bytes")
    return n.value


def pool_workspace_bytes(desc: sp_pool_desc, batch: Batch) -> int:
    n = ctypes.c_size_t()
    _check(lib().sp_pool_workspace_bytes(ctypes.byref(desc), batch.ref(), ctypes.byref(n)),
           "sp_pool_workspace_bytes")
    return n.value


def select_workspace_bytes(batch: Batch, C: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sp_select_workspace_bytes(batch.ref(), C, ctypes.byref(n)),
           "sp_select_workspace_bytes")
    return n.value


def gather_workspace_bytes(batch: Batch, C: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sp_gather_workspace_bytes(batch.ref(), C, ctypes.byref(n)),
           "sp_gather_workspace_bytes")
    return n.value


def sp_score_attention(q: torch.Tensor, k: torch.Tensor, offsets, n_layers: int, n_q_heads: int,
                       n_kv_heads: int, head_dim: int, n_lookahead: int, scale=None,
                       algo="auto", out: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, k_scales=None,
                       prefill_row=False, row_pool=1) -> torch.Tensor:
    """Token importance [sum N_b] fp32 (see the C header for layouts). K may
    be fp8 e4m3 codes with bf16 Q; k_scales ([n_layers * n_kv_heads]) then
    gives each (layer, KV head)'s key scale. prefill_row: q holds
    n_lookahead + 1 steps, the first the prompt's last row."""
    batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
    desc = attn_desc(n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, q.dtype, scale, algo,
                     k_dtype=k.dtype, k_scales=k_scales, prefill_row=prefill_row,
                     row_pool=row_pool)
    steps = n_lookahead + int(bool(prefill_row))
    if not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous")
    if q.dtype != k.dtype and not (q.dtype == torch.bfloat16 and k.dtype == torch.float8_e4m3fn):
        raise ValueError("q and k must share a dtype (or be bf16 Q with fp8 e4m3 K)")
    if q.numel() != batch.B * n_layers * steps * n_q_heads * head_dim:
        raise ValueError("q has the wrong number of elements")
    if k.numel() != n_layers * (batch.total + batch.B * n_lookahead) * n_kv_heads * head_dim:
        raise ValueError("k has the wrong number of elements")
    dev = q.device
    if out is None:
        out = torch.empty(batch.total, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(score_workspace_bytes(desc, batch), dev)
    _check(lib().sp_score_attention(ctypes.byref(desc), batch.ref(), _ptr(q), _ptr(k), _ptr(out),
                                    _ptr(ws), ws.numel(), _stream(dev)), "sp_score_attention")
    return out


def sp_score_attention_noalloc(q: torch.Tensor, k: torch.Tensor, batch: "Batch",
                               desc: sp_attn_desc, out: torch.Tensor) -> torch.Tensor:
    """sp_score_attention_noalloc: the same call with the library's own
    scratch as workspace; allocates nothing (out is the caller's [sum N_b]
    fp32 tensor; desc from attn_desc)."""
    if not (q.is_contiguous() and k.is_contiguous() and out.is_contiguous()):
        raise ValueError("q, k and out must be contiguous")
    if out.dtype != torch.float32 or out.numel() != batch.total:
        raise ValueError("out must be fp32 with one value per prompt token")
    _check(lib().sp_score_attention_noalloc(ctypes.byref(desc), batch.ref(), _ptr(q), _ptr(k),
                                            _ptr(out), _stream(q.device)),
           "sp_score_attention_noalloc")
    return out


def break_even(n_tokens: int, n_kept: int, spec_tps: float = 0.0, target_tps: float = 0.0,
               safety: float = 0.0) -> bool:
    """Whether sparse prefill is estimated to save more than scoring costs
    (sp_break_even; values <= 0 take the defaults 600 t/s, 270 t/s, 1.2)."""
    run = ctypes.c_int32()
    _check(lib().sp_break_even(int(n_tokens), int(n_kept), float(spec_tps), float(target_tps),
                               float(safety), ctypes.byref(run)), "sp_break_even")
    return bool(run.value)


def window_plan(n_tokens: int, window: int, stride: int):
    """(starts, lengths, keep_lengths) of the tool's sliding windows
    (sp_window_plan), as lists."""
    n = ctypes.c_int32()
    lib().sp_window_plan(int(n_tokens), int(window), int(stride), 0, None, None, None,
                         ctypes.byref(n))
    cap = n.value
    starts = (ctypes.c_int64 * cap)()
    lengths, keeps = (ctypes.c_int32 * cap)(), (ctypes.c_int32 * cap)()
    _check(lib().sp_window_plan(int(n_tokens), int(window), int(stride), cap, starts, lengths,
                                keeps, ctypes.byref(n)), "sp_window_plan")
    return list(starts), list(lengths), list(keeps)


def stitch_windows(windows: Batch, starts, keep_lengths, n_tokens: int,
                   window_importance: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Prompt scores [n_tokens] fp32 from the window batch's importance."""
    if out is None:
        out = torch.empty(n_tokens, dtype=torch.float32, device=window_importance.device)
    st = (ctypes.c_int64 * len(starts))(*starts)
    kl = (ctypes.c_int32 * len(keep_lengths))(*keep_lengths)
    _check(lib().sp_stitch_windows(windows.ref(), st, kl, int(n_tokens), _ptr(window_importance),
                                   _ptr(out), _stream(window_importance.device)),
           "sp_stitch_windows")
    return out


def select_legacy_workspace_bytes(batch: Batch, C: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sp_select_legacy_workspace_bytes(batch.ref(), C, ctypes.byref(n)),
           "sp_select_legacy_workspace_bytes")
    return n.value


def select_legacy(batch: Batch, C: int, keep_pct: float, min_tokens: int, max_keep: int,
                  chunk_scores: torch.Tensor, token_ids: torch.Tensor):
    """(kept_ids, kept_pos, kept_offsets) by the tool's legacy rule and cap."""
    dev = chunk_scores.device
    T = batch.total
    kept_ids = torch.empty(T, dtype=torch.int32, device=dev)
    kept_pos = torch.empty(T, dtype=torch.int32, device=dev)
    kept_off = torch.empty(batch.B + 1, dtype=torch.int64, device=dev)
    ws = _ws(select_legacy_workspace_bytes(batch, C), dev)
    _check(lib().sp_select_legacy(batch.ref(), C, float(keep_pct), int(min_tokens), int(max_keep),
                                  _ptr(chunk_scores), _ptr(token_ids), _ptr(kept_ids),
                                  _ptr(kept_pos), _ptr(kept_off), _ptr(ws), ws.numel(),
                                  _stream(dev)), "sp_select_legacy")
    return kept_ids, kept_pos, kept_off


class ScorePlan(NamedTuple):
    kernel: str              # "stream" (single pass) or "two_pass"
    n_launches: int
    prompt_launch: list      # launch index of each prompt


def score_plan(desc: sp_attn_desc, batch: Batch) -> ScorePlan:
    """What sp_score_attention runs for this descriptor and batch on the
    current device (sp_score_plan)."""
    kernel, n = ctypes.c_int32(), ctypes.c_int32()
    per = (ctypes.c_int32 * batch.B)()
    _check(lib().sp_score_plan(ctypes.byref(desc), batch.ref(), ctypes.byref(kernel),
                               ctypes.byref(n), per), "sp_score_plan")
    name = {SP_SCORE_STREAM: "stream", SP_SCORE_TWO_PASS: "two_pass"}[kernel.value]
    return ScorePlan(name, n.value, list(per))


def score_status(ws: torch.Tensor) -> int:
    """Status word of the last finished sp_score_attention on this workspace
    (0 = ok; 1 = a cross-block wait timed out and the importance is invalid)."""
    out = ctypes.c_int32(-1)
    _check(lib().sp_score_status(_ptr(ws), ctypes.byref(out), _stream(ws.device)), "sp_score_status")
    return out.value


def sp_pool_chunk(importance: torch.Tensor, offsets, W=13, C=32, normalize=True, first_n=64,
                  first_mult=1.5, last_n=128, last_mult=1.3, token_scores: bool = True,
                  out_tokens=None, out_chunks=None, ws=None):
    """(token_scores [sum N_b] or None, chunk_scores [sum nc_b]) fp32."""
    batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
    desc = pool_desc(W, C, normalize, first_n, first_mult, last_n, last_mult)
    if importance.dtype != torch.float32 or importance.numel() != batch.total:
        raise ValueError("importance must be fp32 [sum N_b]")
    dev = importance.device
    if token_scores and out_tokens is None:
        out_tokens = torch.empty(batch.total, dtype=torch.float32, device=dev)
    if out_chunks is None:
        out_chunks = torch.empty(batch.n_chunks(C) if C > 0 else 1, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(pool_workspace_bytes(desc, batch), dev)
    _check(lib().sp_pool_chunk(ctypes.byref(desc), batch.ref(), _ptr(importance),
                               _ptr(out_tokens if token_scores else None), _ptr(out_chunks),
                               _ptr(ws), ws.numel(), _stream(dev)), "sp_pool_chunk")
    return (out_tokens if token_scores else None), out_chunks


def sp_select_chunks(chunk_scores: torch.Tensor, offsets, C: int, mode: str, param: float,
                     out_keep=None, out_counts=None, ws=None):
    """(keep [sum nc_b] uint8, n_kept_chunks [B] int32)."""
    batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
    if chunk_scores.dtype != torch.float32:
        raise ValueError("chunk_scores must be fp32")
    dev = chunk_scores.device
    if out_keep is None:
        out_keep = torch.empty(chunk_scores.numel(), dtype=torch.uint8, device=dev)
    if out_counts is None:
        out_counts = torch.empty(batch.B, dtype=torch.int32, device=dev)
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    if ws is None:
        ws = _ws(select_workspace_bytes(batch, C), dev)
    _check(lib().sp_select_chunks(m, float(param), batch.ref(), C, _ptr(chunk_scores),
                                  _ptr(out_keep), _ptr(out_counts), _ptr(ws), ws.numel(),
                                  _stream(dev)), "sp_select_chunks")
    return out_keep, out_counts


def sp_gather_kept(keep: torch.Tensor, token_ids: torch.Tensor, offsets, C: int,
                   out_ids=None, out_pos=None, out_offsets=None, ws=None):
    """(kept_ids [sum N_b] int32, kept_pos [sum N_b] int32, kept_offsets [B+1] int64).

    Only the first kept_offsets[B] entries of kept_ids / kept_pos are written.
    """
    batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
    if token_ids.dtype != torch.int32 or keep.dtype != torch.uint8:
        raise ValueError("token_ids must be int32 and keep uint8")
    dev = token_ids.device
    if out_ids is None:
        out_ids = torch.empty(batch.total, dtype=torch.int32, device=dev)
    if out_pos is None:
        out_pos = torch.empty(batch.total, dtype=torch.int32, device=dev)
    if out_offsets is None:
        out_offsets = torch.empty(batch.B + 1, dtype=torch.int64, device=dev)
    if ws is None:
        ws = _ws(gather_workspace_bytes(batch, C), dev)
    _check(lib().sp_gather_kept(batch.ref(), C, _ptr(keep), _ptr(token_ids), _ptr(out_ids),
                                _ptr(out_pos), _ptr(out_offsets), _ptr(ws), ws.numel(),
                                _stream(dev)), "sp_gather_kept")
    return out_ids, out_pos, out_offsets


def post_workspace_bytes(desc: sp_pool_desc, batch: Batch) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sp_pool_select_gather_workspace_bytes(ctypes.byref(desc), batch.ref(),
                                                       ctypes.byref(n)),
           "sp_pool_select_gather_workspace_bytes")
    return n.value


def post_plan(desc: sp_pool_desc, batch: Batch) -> int:
    """Tokens per block of the one-launch form on the current device (0: the
    call runs the separate kernels)."""
    tb = ctypes.c_int32(-1)
    _check(lib().sp_pool_select_gather_plan(ctypes.byref(desc), batch.ref(), ctypes.byref(tb)),
           "sp_pool_select_gather_plan")
    return tb.value


POST_FORMS = {0: "separate", 1: "grid", 2: "die"}


def post_form(desc: sp_pool_desc, batch: Batch):
    """(form, tokens per block) of sp_pool_select_gather for this batch on the
    current device: form "die" (one launch, each die runs the batch), "grid"
    (one launch over every CU) or "separate" (the three stages' kernels)."""
    form, tb = ctypes.c_int32(-1), ctypes.c_int32(-1)
    _check(lib().sp_pool_select_gather_form(ctypes.byref(desc), batch.ref(), ctypes.byref(form),
                                            ctypes.byref(tb)), "sp_pool_select_gather_form")
    return POST_FORMS[form.value], tb.value


def sp_pool_select_gather(importance: torch.Tensor, token_ids: torch.Tensor, offsets, mode: str,
                          param: float, W=13, C=32, normalize=True, first_n=64, first_mult=1.5,
                          last_n=128, last_mult=1.3, token_scores: bool = True, ws=None):
    """sp_pool_chunk + sp_select_chunks + sp_gather_kept in one call: (token_scores
    or None, chunk_scores, keep, n_kept_chunks, kept_ids, kept_pos, kept_offsets)."""
    batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
    desc = pool_desc(W, C, normalize, first_n, first_mult, last_n, last_mult)
    if importance.dtype != torch.float32 or importance.numel() != batch.total:
        raise ValueError("importance must be fp32 [sum N_b]")
    if token_ids.dtype != torch.int32 or token_ids.numel() != batch.total:
        raise ValueError("token_ids must be int32 [sum N_b]")
    dev = importance.device
    T, nc = batch.total, batch.n_chunks(C) if C > 0 else 1
    ts = torch.empty(T, dtype=torch.float32, device=dev) if token_scores else None
    cs = torch.empty(nc, dtype=torch.float32, device=dev)
    keep = torch.empty(nc, dtype=torch.uint8, device=dev)
    counts = torch.empty(batch.B, dtype=torch.int32, device=dev)
    ids = torch.empty(T, dtype=torch.int32, device=dev)
    pos = torch.empty(T, dtype=torch.int32, device=dev)
    offs = torch.empty(batch.B + 1, dtype=torch.int64, device=dev)
    if ws is None:
        ws = _ws(post_workspace_bytes(desc, batch), dev)
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().sp_pool_select_gather(ctypes.byref(desc), m, float(param), batch.ref(),
                                       _ptr(importance), _ptr(token_ids), _ptr(ts), _ptr(cs),
                                       _ptr(keep), _ptr(counts), _ptr(ids), _ptr(pos), _ptr(offs),
                                       _ptr(ws), ws.numel(), _stream(dev)),
           "sp_pool_select_gather")
    return ts, cs, keep, counts, ids, pos, offs


class Pipeline:
    """The whole path on preallocated buffers (what the benchmark times):
    sp_score_attention, then sp_pool_select_gather (fused=True) or the three
    calls it stands for.

    Holds device buffers for one batch shape; :meth:`run` enqueues the whole
    path on the current stream and returns nothing (results stay in the
    attributes ``importance``, ``token_scores``, ``chunk_scores``, ``keep``,
    ``n_kept``, ``kept_ids``, ``kept_pos``, ``kept_offsets``).
    """

    def __init__(self, offsets, n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, dtype,
                 device, W=13, C=32, normalize=True, boost=True, mode="mass", param=0.85,
                 algo="auto", scale=None, token_scores=True, k_dtype=None, k_scales=None,
                 prefill_row=False, pool_before_max=False, fused=True):
        self.batch = offsets if isinstance(offsets, Batch) else Batch(offsets)
        self.fused = fused
        fm, lm = (1.5, 1.3) if boost else (1.0, 1.0)
        self.adesc = attn_desc(n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, dtype,
                               scale, algo, k_dtype=k_dtype, k_scales=k_scales,
                               prefill_row=prefill_row, row_pool=W if pool_before_max else 1)
        # Pool-before-max pools the probability rows inside the scoring call.
        self.pdesc = pool_desc(1 if pool_before_max else W, C, normalize, 64, fm, 128, lm)
        self.C, self.mode, self.param = C, _MODES[mode], float(param)
        self.shape = (n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead)
        B, T, nc = self.batch.B, self.batch.total, self.batch.n_chunks(C)
        f32 = dict(dtype=torch.float32, device=device)
        self.importance = torch.empty(T, **f32)
        self.token_scores = torch.empty(T, **f32) if token_scores else None
        self.chunk_scores = torch.empty(nc, **f32)
        self.keep = torch.empty(nc, dtype=torch.uint8, device=device)
        self.n_kept = torch.empty(B, dtype=torch.int32, device=device)
        self.kept_ids = torch.empty(T, dtype=torch.int32, device=device)
        self.kept_pos = torch.empty(T, dtype=torch.int32, device=device)
        self.kept_offsets = torch.empty(B + 1, dtype=torch.int64, device=device)
        self.ws_score = _ws(score_workspace_bytes(self.adesc, self.batch), device)
        self.ws_pool = _ws(pool_workspace_bytes(self.pdesc, self.batch), device)
        self.ws_select = _ws(select_workspace_bytes(self.batch, C), device)
        self.ws_gather = _ws(gather_workspace_bytes(self.batch, C), device)
        self.ws_post = _ws(post_workspace_bytes(self.pdesc, self.batch), device)
        self.device = device

    def score_status(self) -> int:
        return score_status(self.ws_score)

    def post_status(self) -> int:
        """Status of the latest sp_pool_select_gather on the pipeline's workspace."""
        return score_status(self.ws_post)

    def run(self, q: torch.Tensor, k: torch.Tensor, token_ids: torch.Tensor, check: bool = False):
        """The path on the pipeline's stream. check=True waits for it and
        raises if a cross-block wait timed out (the results are then invalid)."""
        self.run_score(q, k)
        self.run_post(token_ids)
        if check:
            if self.score_status() != 0:
                raise SpError(SP_ERR_DEVICE, "sp_score_attention (a cross-block wait timed out)")
            if self.fused and self.post_status() != 0:
                raise SpError(SP_ERR_DEVICE, "sp_pool_select_gather (a cross-block wait timed out)")

    def run_score(self, q: torch.Tensor, k: torch.Tensor):
        """The scoring call alone (importance from Q and K)."""
        _check(lib().sp_score_attention(ctypes.byref(self.adesc), self.batch.ref(), _ptr(q), _ptr(k),
                                        _ptr(self.importance), _ptr(self.ws_score),
                                        self.ws_score.numel(), _stream(self.device)),
               "sp_score_attention")

    def run_post(self, token_ids: torch.Tensor):
        """The stages after scoring, on the pipeline's importance."""
        L = lib()
        st = _stream(self.device)
        b = self.batch.ref()
        if self.fused:
            _check(L.sp_pool_select_gather(
                ctypes.byref(self.pdesc), self.mode, self.param, b, _ptr(self.importance),
                _ptr(token_ids), _ptr(self.token_scores), _ptr(self.chunk_scores), _ptr(self.keep),
                _ptr(self.n_kept), _ptr(self.kept_ids), _ptr(self.kept_pos),
                _ptr(self.kept_offsets), _ptr(self.ws_post), self.ws_post.numel(), st),
                "sp_pool_select_gather")
            return
        _check(L.sp_pool_chunk(ctypes.byref(self.pdesc), b, _ptr(self.importance),
                               _ptr(self.token_scores), _ptr(self.chunk_scores),
                               _ptr(self.ws_pool), self.ws_pool.numel(), st), "sp_pool_chunk")
        _check(L.sp_select_chunks(self.mode, self.param, b, self.C, _ptr(self.chunk_scores),
                                  _ptr(self.keep), _ptr(self.n_kept), _ptr(self.ws_select),
                                  self.ws_select.numel(), st),
               "sp_select_chunks")
        _check(L.sp_gather_kept(b, self.C, _ptr(self.keep), _ptr(token_ids), _ptr(self.kept_ids),
                                _ptr(self.kept_pos), _ptr(self.kept_offsets),
                                _ptr(self.ws_gather), self.ws_gather.numel(), st),
               "sp_gather_kept")


class ToolPipeline:
    """The standalone tool's path for one prompt: the windows of
    sp_window_plan scored as one batch, stitched, pooled/normalised/boosted,
    then the legacy chunk rule with its cap. Buffers are preallocated."""

    def __init__(self, n_tokens, window, stride, n_layers, n_q_heads, n_kv_heads, head_dim,
                 n_lookahead, dtype, device, C=32, W=1, normalize=True, boost=True,
                 keep_pct=0.3, min_tokens=128, max_keep=2000, prefill_row=True, algo="auto"):
        self.n = int(n_tokens)
        self.starts, self.lengths, self.keeps = window_plan(n_tokens, window, stride)
        self.windows = Batch(np.concatenate([[0], np.cumsum(self.lengths)]))
        self.batch = self.windows          # the batch sp_score_attention scores
        self.prompt = Batch([0, self.n])
        fm, lm = (1.5, 1.3) if boost else (1.0, 1.0)
        self.adesc = attn_desc(n_layers, n_q_heads, n_kv_heads, head_dim, n_lookahead, dtype,
                               None, algo, prefill_row=prefill_row)
        self.pdesc = pool_desc(W, C, normalize, 64, fm, 128, lm)
        self.C, self.keep_pct, self.min_tokens, self.max_keep = C, keep_pct, min_tokens, max_keep
        f32 = dict(dtype=torch.float32, device=device)
        self.importance = torch.empty(self.windows.total, **f32)
        self.scores = torch.empty(self.n, **f32)
        self.token_scores = torch.empty(self.n, **f32)
        self.chunk_scores = torch.empty(self.prompt.n_chunks(C), **f32)
        self.kept_ids = torch.empty(self.n, dtype=torch.int32, device=device)
        self.kept_pos = torch.empty(self.n, dtype=torch.int32, device=device)
        self.kept_offsets = torch.empty(2, dtype=torch.int64, device=device)
        self.ws_score = _ws(score_workspace_bytes(self.adesc, self.windows), device)
        self.ws_pool = _ws(pool_workspace_bytes(self.pdesc, self.prompt), device)
        self.ws_legacy = _ws(select_legacy_workspace_bytes(self.prompt, C), device)
        self._starts = (ctypes.c_int64 * len(self.starts))(*self.starts)
        self._keeps = (ctypes.c_int32 * len(self.keeps))(*self.keeps)
        self.device = device

    def score_status(self) -> int:
        return score_status(self.ws_score)

    def run(self, q: torch.Tensor, k: torch.Tensor, token_ids: torch.Tensor, check: bool = False):
        """q, k: the window batch's Q and K; token_ids: [n_tokens] of the prompt.
        check=True waits and raises if a scoring wait timed out."""
        self.run_score(q, k)
        self.run_post(token_ids)
        if check and self.score_status() != 0:
            raise SpError(SP_ERR_DEVICE, "sp_score_attention (a cross-block wait timed out)")

    def run_score(self, q: torch.Tensor, k: torch.Tensor):
        """The scoring call on the window batch alone."""
        _check(lib().sp_score_attention(ctypes.byref(self.adesc), self.windows.ref(), _ptr(q),
                                        _ptr(k), _ptr(self.importance), _ptr(self.ws_score),
                                        self.ws_score.numel(), _stream(self.device)),
               "sp_score_attention")

    def run_post(self, token_ids: torch.Tensor):
        """Stitching, pooling and the legacy selection on the window scores."""
        L = lib()
        st = _stream(self.device)
        _check(L.sp_stitch_windows(self.windows.ref(), self._starts, self._keeps, self.n,
                                   _ptr(self.importance), _ptr(self.scores), st),
               "sp_stitch_windows")
        _check(L.sp_pool_chunk(ctypes.byref(self.pdesc), self.prompt.ref(), _ptr(self.scores),
                               _ptr(self.token_scores), _ptr(self.chunk_scores),
                               _ptr(self.ws_pool), self.ws_pool.numel(), st), "sp_pool_chunk")
        _check(L.sp_select_legacy(self.prompt.ref(), self.C, float(self.keep_pct),
                                  int(self.min_tokens), int(self.max_keep), _ptr(self.chunk_scores),
                                  _ptr(token_ids), _ptr(self.kept_ids), _ptr(self.kept_pos),
                                  _ptr(self.kept_offsets), _ptr(self.ws_legacy),
                                  self.ws_legacy.numel(), st), "sp_select_legacy")
