"""CPU oracle of the token-importance path (ctypes wrapper over sp_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the library. The arithmetic lives in
``sp_oracle.c`` (plain fp64 loops); this wrapper only marshals arrays.

Parity status of each function (what pins it, beyond itself):

* ``importance``: closed forms (all-zero Q, a single hot key, a hot
  lookahead key that only later queries see), row sums, brute force against
  a numpy softmax on tiny shapes, permutation invariants.
* ``pool_chunk``: identity at W=1, constants, impulses, numpy convolution,
  hand-computed boosts and normalisation.
* ``select_top_p`` / ``select_mass``: exhaustive subset search on small
  chunk counts, and the kept-token counts printed in the pull request's
  stress tables (``tests/golden/pr_kept_counts.txt``).
* ``gather``: brute-force list construction.

End-to-end scores on large random inputs have no printed values on the
pages; there they rest on the pins above.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsp_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into ``oracle/libsp_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_softmax_row.argtypes = [ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         _fp, _fp,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp,
                                         _dp]
        L.oracle_importance.argtypes = [ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, _fp, _fp, _dp,
                                        ctypes.c_int, _dp]
        L.oracle_pool_chunk.argtypes = [ctypes.c_int64, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                        _dp, _dp]
        L.oracle_top_p_count.argtypes = [ctypes.c_int64, ctypes.c_double]
        L.oracle_top_p_count.restype = ctypes.c_int64
        L.oracle_select_top_p.argtypes = [ctypes.c_int64, _dp, ctypes.c_double, _u8p]
        L.oracle_select_top_p.restype = ctypes.c_int64
        L.oracle_select_mass.argtypes = [ctypes.c_int64, _dp, ctypes.c_double, _u8p]
        L.oracle_select_mass.restype = ctypes.c_int64
        L.oracle_gather.argtypes = [ctypes.c_int64, ctypes.c_int, _u8p, _i32p, _i32p, _i32p]
        L.oracle_gather.restype = ctypes.c_int64
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def _as_f32(x) -> np.ndarray:
    """Widen Q/K to a contiguous fp32 numpy array (exact for bf16 and fp8 input)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _scales(k_scales, n):
    """Key scales as an fp64 array of n values, or None (keys are values)."""
    if k_scales is None:
        return None
    try:
        import torch
        if isinstance(k_scales, torch.Tensor):
            k_scales = k_scales.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    ks = np.ascontiguousarray(np.asarray(k_scales, dtype=np.float64).reshape(-1))
    assert ks.size == n, "k_scales needs one value per (layer, KV head)"
    return ks


def softmax_row(offsets, q, k, n_layers, Hq, Hkv, d, L, scale, b, l, j, h,
                k_scales=None, prefill_row=False) -> np.ndarray:
    """Softmax probabilities of query (b, l, j, h) over its N_b - pre + j + 1
    visible keys (L lookahead keys; with prefill_row, q has L + 1 steps and
    step 0 is the prompt's last row); with k_scales, K holds codes and
    key = k_scales[l][g] * code."""
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    qf, kf = _as_f32(q), _as_f32(k)
    ks = _scales(k_scales, n_layers * Hkv)
    n = int(off[b + 1] - off[b])
    pre = int(bool(prefill_row))
    p = np.empty(max(n - pre + j + 1, 1), dtype=np.float64)
    rc = lib().oracle_softmax_row(len(off) - 1, _ptr(off, _i64p), n_layers, Hq, Hkv, d, L, pre,
                                  scale,
                                  _ptr(qf, _fp), _ptr(kf, _fp), b, l, j, h, _ptr(p, _dp),
                                  None if ks is None else _ptr(ks, _dp))
    if rc != 0:
        raise ValueError("oracle_softmax_row: bad arguments")
    return p


def importance(offsets, q, k, n_layers, Hq, Hkv, d, L, scale, nthreads: int = 0,
               k_scales=None, prefill_row=False, row_pool: int = 1) -> np.ndarray:
    """Importance of every prompt token, [sum N_b] fp64 (k_scales and
    prefill_row: see softmax_row). row_pool = W > 1 pools every probability
    row's prompt columns (centred, width W) before the max over heads and
    layers."""
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    qf, kf = _as_f32(q), _as_f32(k)
    ks = _scales(k_scales, n_layers * Hkv)
    B = len(off) - 1
    pre = int(bool(prefill_row))
    assert qf.size == B * n_layers * (L + pre) * Hq * d, "q has the wrong size"
    assert kf.size == n_layers * (int(off[-1]) + B * L) * Hkv * d, "k has the wrong size"
    imp = np.empty(int(off[-1]), dtype=np.float64)
    rc = lib().oracle_importance(B, _ptr(off, _i64p), n_layers, Hq, Hkv, d, L, pre, row_pool, scale,
                                 _ptr(qf, _fp), _ptr(kf, _fp), _ptr(imp, _dp), nthreads,
                                 None if ks is None else _ptr(ks, _dp))
    if rc != 0:
        raise ValueError("oracle_importance: bad arguments")
    return imp


def pool_chunk(imp, W=13, C=32, normalize=True, first_n=64, first_mult=1.5,
               last_n=128, last_mult=1.3):
    """(token_scores [n], chunk_scores [ceil(n/C)]) of one prompt, fp64."""
    x = np.ascontiguousarray(np.asarray(imp, dtype=np.float64))
    n = x.size
    nc = (n + C - 1) // C if C >= 1 else 1
    ts = np.empty(n, dtype=np.float64)
    cs = np.empty(nc, dtype=np.float64)
    rc = lib().oracle_pool_chunk(n, _ptr(x, _dp), W, C, int(bool(normalize)), first_n, first_mult,
                                 last_n, last_mult, _ptr(ts, _dp), _ptr(cs, _dp))
    if rc != 0:
        raise ValueError("oracle_pool_chunk: bad arguments")
    return ts, cs


def top_p_count(nc: int, p: float) -> int:
    return int(lib().oracle_top_p_count(nc, p))


def select(chunk_scores, mode: str, param: float) -> np.ndarray:
    """Keep flags [nc] (uint8) of one prompt; mode is 'top_p' or 'mass'."""
    cs = np.ascontiguousarray(np.asarray(chunk_scores, dtype=np.float64))
    keep = np.zeros(cs.size, dtype=np.uint8)
    fn = {"top_p": lib().oracle_select_top_p, "mass": lib().oracle_select_mass}[mode]
    rc = fn(cs.size, _ptr(cs, _dp), float(param), _ptr(keep, _u8p))
    if rc < 0:
        raise ValueError("oracle select: bad arguments")
    return keep


def gather(keep, ids, C=32):
    """(kept_ids, kept_pos) of one prompt."""
    kp = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8))
    idv = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    n = idv.size
    out_i = np.empty(n, dtype=np.int32)
    out_p = np.empty(n, dtype=np.int32)
    w = lib().oracle_gather(n, C, _ptr(kp, _u8p), _ptr(idv, _i32p), _ptr(out_i, _i32p),
                            _ptr(out_p, _i32p))
    if w < 0:
        raise ValueError("oracle_gather: bad arguments")
    return out_i[:w].copy(), out_p[:w].copy()


def pipeline(inputs, mode: str = None, param: float = None, nthreads: int = 0, imp=None):
    """Whole path on a ``workloads.Inputs``: per-prompt results as a dict of lists."""
    w = inputs.workload
    if mode is None:
        mode, param = w.select
    # Pool-before-max pools the probability rows, and then not again.
    row_pool, W = (w.pool_window, 1) if w.pool_before_max else (1, w.pool_window)
    if imp is None:
        imp = importance(inputs.offsets.numpy(), inputs.q, inputs.k, w.n_layers, w.n_q_heads,
                         w.n_kv_heads, w.head_dim, w.n_lookahead, inputs.scale, nthreads,
                         k_scales=inputs.k_scales, prefill_row=w.prefill_row, row_pool=row_pool)
    off = inputs.offsets.numpy()
    ids = inputs.token_ids.numpy()
    fm, lm = (1.5, 1.3) if w.boost else (1.0, 1.0)
    out = {"imp": imp, "token_scores": [], "chunk_scores": [], "keep": [], "kept_ids": [],
           "kept_pos": []}
    for b in range(len(off) - 1):
        x = imp[off[b]:off[b + 1]]
        ts, cs = pool_chunk(x, W, w.chunk_size, w.normalize, 64, fm, 128, lm)
        keep = select(cs, mode, param)
        ki, kp = gather(keep, ids[off[b]:off[b + 1]], w.chunk_size)
        out["token_scores"].append(ts)
        out["chunk_scores"].append(cs)
        out["keep"].append(keep)
        out["kept_ids"].append(ki)
        out["kept_pos"].append(kp)
    return out


def break_even(n_tokens: int, n_kept: int, spec_tps: float = 600.0, target_tps: float = 270.0,
               safety: float = 1.2) -> bool:
    """Break-even gate, "SpecPrefill — Implementation Guide", v3 Improvements
    item 4 and Configuration Reference: scoring is estimated at n_tokens at the
    speculator's rate, the saving at the dropped tokens at the target's rate;
    sparse prefill runs unless the saving is below the scoring time times the
    safety factor."""
    scoring_time = n_tokens / spec_tps
    saved_time = (n_tokens - n_kept) / target_tps
    return not (saved_time < scoring_time * safety)


# ----------------------------------------------------------------------------
# Standalone-tool semantics: sliding windows, legacy chunk selection, thinning
# ("SpecPrefill — Implementation Guide": Sliding Window, v3.1 Optimizations &
# Bug Fixes items 6-7, Sliding Window Loop (v3.1 — fixed), Configuration
# Reference, and the chunk-selection and main-loop parts of Full Source Code).
# ----------------------------------------------------------------------------

def window_plan(n_tokens: int, window: int, stride: int):
    """Windows of the v3.1 loop as (start, length, keep) triples.

    A window starts at pos (0, then every stride) and spans
    min(window, n_tokens - pos) tokens. It is the last one when it reaches
    the end of the prompt or when the next start would (pos + stride >=
    n_tokens); the loop stops after it. Every window keeps the scores of
    its first `stride` tokens, the last one keeps all of its tokens.
    """
    assert n_tokens >= 1 and window >= 1 and 1 <= stride <= window
    plan, pos = [], 0
    while pos < n_tokens:
        end = min(pos + window, n_tokens)
        last = end >= n_tokens or pos + stride >= n_tokens
        plan.append((pos, end - pos, end - pos if last else stride))
        if last:
            break
        pos += stride
    return plan


def stitch(plan, window_scores, n_tokens: int) -> np.ndarray:
    """Prompt scores from per-window scores: each window adds its kept
    tokens' scores, overlaps are averaged, and a token no window scored gets
    1.0 (the guide's default)."""
    acc = np.zeros(n_tokens)
    cnt = np.zeros(n_tokens, dtype=np.int64)
    for (start, length, keep), ws in zip(plan, window_scores):
        ws = np.asarray(ws, dtype=np.float64)
        assert ws.size == length
        acc[start:start + keep] += ws[:keep]
        cnt[start:start + keep] += 1
    out = np.ones(n_tokens)
    m = cnt > 0
    out[m] = acc[m] / cnt[m]
    return out


def legacy_keep_count(n_chunks: int, keep_pct: float) -> int:
    """Chunks the legacy rule ranks in: ceil(n_chunks * keep_pct), at least
    one, with the fraction and the product in single precision (the tool
    reads the fraction into a float)."""
    prod = np.float32(n_chunks) * np.float32(keep_pct)
    return max(1, int(math.ceil(float(prod))))


def select_legacy(scores, chunk_size: int = 32, keep_pct: float = 0.3,
                  min_tokens: int = 128) -> np.ndarray:
    """Kept token indices, ascending, by the standalone tool's chunk rule:
    chunk means over the tokens each chunk holds (sums in double, the mean
    rounded to single precision), then select_legacy_from_means."""
    x = np.asarray(scores, dtype=np.float64)
    n = x.size
    nc = (n + chunk_size - 1) // chunk_size
    means = np.array([np.float32(x[c * chunk_size:min(n, (c + 1) * chunk_size)].sum()
                                 / (min(n, (c + 1) * chunk_size) - c * chunk_size))
                      for c in range(nc)], dtype=np.float32)
    return select_legacy_from_means(means, n, chunk_size, keep_pct, min_tokens)


def select_legacy_from_means(means, n: int, chunk_size: int = 32, keep_pct: float = 0.3,
                             min_tokens: int = 128) -> np.ndarray:
    """The legacy rule on given chunk means (single precision) of an n-token
    prompt.

    - effective minimum: min(min_tokens, max(4, n // 10)); if keep_pct >= 1
      or the prompt is no longer than it, every token is kept;
    - threshold: the kc-th largest chunk mean (kc from legacy_keep_count);
      every chunk whose mean reaches it is kept, ties included;
    - tokens 0-3 and, when there are more than 4 tokens, the last two are
      always kept;
    - while fewer than the effective minimum are kept, tokens of the chunks
      below the threshold are added in index order.
    """
    means = np.asarray(means, dtype=np.float32)
    nc = means.size
    assert nc == (n + chunk_size - 1) // chunk_size
    eff_min = min(min_tokens, max(4, n // 10))
    if keep_pct >= 1.0 or n <= eff_min:
        return np.arange(n, dtype=np.int64)
    kc = legacy_keep_count(nc, keep_pct)
    th = np.sort(means)[::-1][kc - 1]
    kept = set()
    for c in range(nc):
        if means[c] >= th:
            kept.update(range(c * chunk_size, min(n, (c + 1) * chunk_size)))
    always = [0, 1, 2, 3] + ([n - 2, n - 1] if n > 4 else [])
    kept.update(a for a in always if a < n)
    for c in range(nc):
        if len(kept) >= eff_min:
            break
        if means[c] < th:
            for t in range(c * chunk_size, min(n, (c + 1) * chunk_size)):
                if len(kept) >= eff_min:
                    break
                kept.add(t)
    return np.array(sorted(kept), dtype=np.int64)


def thin(kept, max_keep: int) -> np.ndarray:
    """The tool's cap on tokens sent to the target: above max_keep kept
    tokens, keep every step-th one (step = count // max_keep) up to max_keep
    of them, the last of which is replaced by the final kept token."""
    kept = np.asarray(kept, dtype=np.int64)
    k = kept.size
    if k <= max_keep:
        return kept.copy()
    step = k // max_keep
    out = kept[::step][:max_keep].copy()
    out[-1] = kept[-1]
    return out


def tool_pipeline(win_inputs, plan, nthreads: int = 0):
    """The standalone tool on a ``workloads.WindowInputs``: window importance,
    stitched prompt scores, token scores (normalised and boosted, no pooling
    unless the workload asks), the legacy kept tokens and the capped list."""
    w = win_inputs.workload
    bi = win_inputs.batch
    imp = importance(bi.offsets.numpy(), bi.q, bi.k, w.n_layers, w.n_q_heads, w.n_kv_heads,
                     w.head_dim, w.n_lookahead, bi.scale, nthreads, prefill_row=w.prefill_row)
    off = bi.offsets.numpy()
    per_window = [imp[off[i]:off[i + 1]] for i in range(len(plan))]
    scores = stitch(plan, per_window, win_inputs.n_tokens)
    fm, lm = (1.5, 1.3) if w.boost else (1.0, 1.0)
    ts, cs = pool_chunk(scores, w.pool_window, w.chunk_size, w.normalize, 64, fm, 128, lm)
    kept = select_legacy(ts, w.chunk_size, w.keep_pct, w.min_tokens)
    final = thin(kept, w.max_keep)
    ids = win_inputs.token_ids.numpy()
    return {"imp": imp, "scores": scores, "token_scores": ts, "chunk_scores": cs, "kept": kept,
            "final": final, "final_ids": ids[final]}
