"""Seeded synthetic inputs for the token-importance path.

This module only draws random tensors and builds the input layout. It holds
none of the method's arithmetic, so both the oracle tests and the HIP path
can take their inputs from it.

What the inputs stand in for: the pages measure on real prompts (needle
retrieval, RULER-style suites, LongBench QA, hand-made stress prompts) fed to
a real draft model. Neither the prompts nor the draft weights are available,
so each workload is a seeded draw with the shapes of those runs:

* Q (the lookahead queries) and K (the draft KV cache) are N(0, 1).
* "Planted" spans are 32-token, chunk-aligned runs of keys that are pushed
  towards the mean query direction of their KV group, so the draft attends to
  them; they play the role of the needle / evidence chunks.
* Token ids are uniform in [0, 2**17).
* Quantised-K workloads (``k_fp8``) store K as fp8 e4m3 codes with one fp32
  scale per (layer, KV head): scale = max |K| / 448 over that slice (the
  largest finite e4m3 value), code = K / scale rounded to e4m3. This stands
  in for a draft model whose K cache is kept in an 8-bit type.

Layouts (all C-contiguous):

* ``q``: ``[B][layers][L][Hq][d]``
* ``k``: ``[layers][sum_b (N_b + L)][Hkv][d]``; prompt ``b``'s key rows start
  at ``offsets[b] + b * L`` and hold its ``N_b`` prompt keys followed by its
  ``L`` lookahead keys.
* ``token_ids``: ``[sum_b N_b]`` int32.
* ``offsets``: ``[B + 1]`` int64 prompt-token offsets.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

__all__ = ["Workload", "Inputs", "WORKLOADS", "make_inputs", "small_workload", "quantize_fp8"]

VOCAB = 1 << 17


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic workload (shapes, planting and selection settings)."""

    name: str
    lengths: Optional[tuple]          # prompt lengths; None -> drawn (ragged)
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_lookahead: int
    dtype: torch.dtype
    seed: int
    n_spans: Optional[int]            # per prompt; None -> floor(N / 2048)
    span_strength: Optional[float]    # fixed strength, or None -> U(0.5, 3)
    pool_window: int = 13
    chunk_size: int = 32
    normalize: bool = True
    boost: bool = True
    select: tuple = ("mass", 0.85)    # ("top_p", p) or ("mass", m); first is primary
    also_select: tuple = ()           # further (mode, param) pairs on the same scores
    ragged_count: int = 0             # >0: draw this many lengths log-uniform
    ragged_range: tuple = (2048, 65536)
    k_fp8: bool = False               # K as fp8 e4m3 codes + per-(layer, KV head) scales
    prefill_row: bool = False         # one more query step: the prompt's last row
    pool_before_max: bool = False     # pool each probability row before the head/layer max
    window: int = 0                   # >0: the standalone tool's sliding windows of this size
    stride: int = 0                   # their stride
    keep_pct: float = 0.3             # legacy chunk rule: fraction of chunks
    min_tokens: int = 128             # legacy chunk rule: kept-token floor
    max_keep: int = 2000              # cap on tokens sent to the target

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def steps(self) -> int:
        """Query steps per (layer, head): the lookahead ones, plus the prefill row."""
        return self.n_lookahead + int(self.prefill_row)


WORKLOADS = {
    # 800-token prompt, fp32, 3 planted spans of strength 2, top-p 0.15.
    "n800_fp32": Workload("n800_fp32", (800,), 6, 8, 2, 64, 8, torch.float32,
                          1001, 3, 2.0, normalize=False, boost=False,
                          select=("top_p", 0.15)),
    # 3212-token prompt, bf16, 5 spans of strength 2, top-p 0.30.
    "n3212_bf16": Workload("n3212_bf16", (3212,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1002, 5, 2.0,
                           select=("top_p", 0.30), also_select=(("mass", 0.85),)),
    # 32768-token prompt, 20 spans of varied strength, mass 0.85.
    "n32k_bf16": Workload("n32k_bf16", (32768,), 6, 16, 4, 128, 8,
                          torch.bfloat16, 1003, 20, None,
                          also_select=(("top_p", 0.15),)),
    # 131072-token prompt, 64 spans of varied strength, mass 0.85.
    "n128k_bf16": Workload("n128k_bf16", (131072,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1004, 64, None,
                           also_select=(("top_p", 0.15),)),
    # Same prompt length with no planted spans (diffuse attention).
    "n128k_diffuse_bf16": Workload("n128k_diffuse_bf16", (131072,), 6, 16, 4,
                                   128, 8, torch.bfloat16, 1014, 0, None),
    # A 163840-token prompt (the ~150K-token contexts the PR discussion runs),
    # 80 spans of varied strength: the longest single prompt the single-pass
    # kernel takes in one launch (248 blocks x 21 tiles of 32 keys).
    "n160k_bf16": Workload("n160k_bf16", (163840,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1016, 80, None,
                           also_select=(("top_p", 0.15),)),
    "n160k_fp8k": Workload("n160k_fp8k", (163840,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1016, 80, None, k_fp8=True),
    # Ragged batch: 16 prompts, log-uniform lengths in [2048, 65536].
    "ragged16_bf16": Workload("ragged16_bf16", None, 8, 32, 8, 128, 8,
                              torch.bfloat16, 1500, None, None,
                              select=("top_p", 0.15),
                              also_select=(("mass", 0.85),), ragged_count=16),
    # The same shapes with K quantised to fp8 e4m3 (Q stays bf16).
    "n3212_fp8k": Workload("n3212_fp8k", (3212,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1002, 5, 2.0, select=("top_p", 0.30),
                           also_select=(("mass", 0.85),), k_fp8=True),
    "n128k_fp8k": Workload("n128k_fp8k", (131072,), 6, 16, 4, 128, 8,
                           torch.bfloat16, 1004, 64, None, k_fp8=True),
    # The prefill's last row as one more step: 7 lookahead steps + 1 = 8 rows
    # per head, so the 32 query rows of a KV group stay filled.
    "n3212_prerow_bf16": Workload("n3212_prerow_bf16", (3212,), 6, 16, 4, 128, 7,
                                  torch.bfloat16, 1002, 5, 2.0, select=("top_p", 0.30),
                                  also_select=(("mass", 0.85),), prefill_row=True),
    "n32k_prerow_bf16": Workload("n32k_prerow_bf16", (32768,), 6, 16, 4, 128, 7,
                                 torch.bfloat16, 1003, 20, None,
                                 also_select=(("top_p", 0.15),), prefill_row=True),
    # Pool-before-max: the W = 13 pool moves onto every probability row.
    "n3212_poolmax_bf16": Workload("n3212_poolmax_bf16", (3212,), 6, 16, 4, 128, 8,
                                   torch.bfloat16, 1002, 5, 2.0, select=("top_p", 0.30),
                                   also_select=(("mass", 0.85),), pool_before_max=True),
    "n128k_poolmax_bf16": Workload("n128k_poolmax_bf16", (131072,), 6, 16, 4, 128, 8,
                                   torch.bfloat16, 1004, 64, None,
                                   also_select=(("top_p", 0.15),), pool_before_max=True),
    # The standalone tool: sliding windows (each a separate draft pass with the
    # prefill's last row as a step and 2 lookahead steps), scores stitched,
    # normalised and boosted, then the legacy chunk rule and the 2000-token cap.
    # 4471 tokens in windows of 2000 at stride 1000: the guide's worked example.
    "tool4471_bf16": Workload("tool4471_bf16", (4471,), 6, 16, 4, 128, 2, torch.bfloat16,
                              1601, 5, 2.0, pool_window=1, select=("legacy", 0.3),
                              prefill_row=True, window=2000, stride=1000),
    "tool128k_bf16": Workload("tool128k_bf16", (131072,), 6, 16, 4, 128, 2, torch.bfloat16,
                              1602, 64, None, pool_window=1, select=("legacy", 0.3),
                              prefill_row=True, window=8192, stride=4096),
}


@dataclasses.dataclass
class Inputs:
    workload: Workload
    lengths: List[int]
    offsets: torch.Tensor      # [B+1] int64
    q: torch.Tensor            # [B][layers][S][Hq][d], S = L (+ 1 with the prefill row)
    k: torch.Tensor            # [layers][sum(N_b+L)][Hkv][d]
    token_ids: torch.Tensor    # [sum N_b] int32
    spans: List[List[int]]     # planted chunk indices per prompt
    strengths: List[List[float]]
    k_scales: Optional[torch.Tensor] = None   # [layers][Hkv] fp32 when K holds fp8 codes

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.workload.head_dim)

    @property
    def key_offsets(self) -> List[int]:
        L = self.workload.n_lookahead
        return [int(self.offsets[b]) + b * L for b in range(len(self.lengths) + 1)]


def ragged_lengths(w: Workload) -> List[int]:
    """Prompt lengths for a ragged batch: log-uniform draw from ``w.seed``."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    lo, hi = w.ragged_range
    u = torch.rand(w.ragged_count, generator=g, dtype=torch.float64)
    return [int(round(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo)))))
            for x in u]


def _draw_prompt(w: Workload, n: int, seed: int, k_out: torch.Tensor, q_out: torch.Tensor,
                 n_spans: int):
    """Draw one prompt's Q, K (written into the given slices) and token ids."""
    L, S, Hq, Hkv, d, G = w.n_lookahead, w.steps, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    g = torch.Generator("cpu").manual_seed(seed)
    # Chunks wholly inside [64, n - 128): clear of the boosted edges and of
    # the always-kept final chunk.
    first = 2
    last = (n - 128) // 32 - 1
    eligible = max(0, last - first + 1)
    n_spans = min(n_spans, eligible)
    perm = torch.randperm(eligible, generator=g)[:n_spans] if eligible > 0 else torch.empty(0, dtype=torch.long)
    spans = sorted(int(first + c) for c in perm)
    if w.span_strength is None:
        strengths = (0.5 + 2.5 * torch.rand(n_spans, generator=g, dtype=torch.float64)).tolist()
    else:
        strengths = [float(w.span_strength)] * n_spans
    for layer in range(w.n_layers):
        q = torch.randn(S, Hq, d, generator=g, dtype=torch.float32)
        kk = torch.randn(n + L, Hkv, d, generator=g, dtype=torch.float32)
        for grp in range(Hkv):
            v = q[:, grp * G:(grp + 1) * G, :].reshape(-1, d).mean(dim=0)
            u = v / v.norm()
            for c, s in zip(spans, strengths):
                kk[32 * c:32 * c + 32, grp, :] += float(s) * u
        q_out[layer].copy_(q.to(q_out.dtype))
        k_out[layer].copy_(kk.to(k_out.dtype))
    ids = torch.randint(0, VOCAB, (n,), generator=g, dtype=torch.int64).to(torch.int32)
    return ids, spans, strengths


def make_inputs(w: Workload, lengths: Optional[List[int]] = None) -> Inputs:
    """Build the seeded inputs of workload ``w``.

    ``lengths`` overrides the prompt lengths (used for small parity cases of
    the same shape family); prompt ``b`` draws from seed ``w.seed + b`` in a
    ragged batch and from ``w.seed`` for a single prompt.
    """
    if lengths is None:
        lengths = list(w.lengths) if w.lengths is not None else ragged_lengths(w)
    B = len(lengths)
    L = w.n_lookahead
    offsets = torch.zeros(B + 1, dtype=torch.int64)
    for b, n in enumerate(lengths):
        offsets[b + 1] = offsets[b] + n
    total_keys = int(offsets[-1]) + B * L
    q = torch.empty(B, w.n_layers, w.steps, w.n_q_heads, w.head_dim, dtype=w.dtype)
    k = torch.empty(w.n_layers, total_keys, w.n_kv_heads, w.head_dim,
                    dtype=torch.float32 if w.k_fp8 else w.dtype)
    ids, spans, strengths = [], [], []
    for b, n in enumerate(lengths):
        kb = int(offsets[b]) + b * L
        seed = w.seed + b if B > 1 or w.ragged_count else w.seed
        ns = w.n_spans if w.n_spans is not None else n // 2048
        i, s, st = _draw_prompt(w, n, seed, k[:, kb:kb + n + L], q[b], ns)
        ids.append(i)
        spans.append(s)
        strengths.append(st)
    token_ids = torch.cat(ids) if ids else torch.empty(0, dtype=torch.int32)
    k_scales = None
    if w.k_fp8:
        k, k_scales = quantize_fp8(k)
    return Inputs(w, list(lengths), offsets, q, k, token_ids, spans, strengths, k_scales)


FP8_MAX = 448.0   # largest finite float8 e4m3 (OCP E4M3FN) value


def quantize_fp8(k: torch.Tensor):
    """fp32 K [layers][keys][Hkv][d] -> (fp8 e4m3 codes, [layers][Hkv] fp32
    scales) with scale = max |K| / 448 per (layer, KV head)."""
    amax = k.abs().amax(dim=(1, 3))                       # [layers][Hkv]
    scales = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (k / scales[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.contiguous(), scales.contiguous()


def small_workload(base: str, **overrides) -> Workload:
    """A copy of a named workload with some fields replaced (small cases)."""
    return dataclasses.replace(WORKLOADS[base], **overrides)


@dataclasses.dataclass
class WindowInputs:
    """Inputs of the standalone tool's windows: every window is a prompt of
    its own for the draft model (fresh context), so each one draws its own Q
    and K; the planted spans and the token ids belong to the whole prompt."""
    workload: Workload
    n_tokens: int
    starts: List[int]
    batch: Inputs              # the windows as a batch of prompts
    token_ids: torch.Tensor    # [n_tokens] int32, the whole prompt's ids
    spans: List[int]           # planted chunk indices of the whole prompt
    strengths: List[float]


def make_window_inputs(w: Workload, starts: List[int], lengths: List[int]) -> WindowInputs:
    """Seeded inputs for windows at the given starts and lengths (the caller
    supplies the window plan). Window i draws Q [layers][S][Hq][d] and K
    [layers][len_i + L][Hkv][d] from N(0, 1) with seed w.seed + 7919 * (i + 1);
    a planted span adds s * u to the K rows of its tokens inside the window
    (u: the unit mean query of the group in that window and layer)."""
    n = int(w.lengths[0])
    L, S, Hq, Hkv, d, G = w.n_lookahead, w.steps, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    g = torch.Generator("cpu").manual_seed(w.seed)
    first, last = 2, (n - 128) // 32 - 1
    eligible = max(0, last - first + 1)
    ns = min(w.n_spans if w.n_spans is not None else n // 2048, eligible)
    perm = torch.randperm(eligible, generator=g)[:ns] if eligible > 0 else torch.empty(0, dtype=torch.long)
    spans = sorted(int(first + c) for c in perm)
    if w.span_strength is None:
        strengths = (0.5 + 2.5 * torch.rand(ns, generator=g, dtype=torch.float64)).tolist()
    else:
        strengths = [float(w.span_strength)] * ns
    ids = torch.randint(0, VOCAB, (n,), generator=g, dtype=torch.int64).to(torch.int32)
    B = len(starts)
    offsets = torch.zeros(B + 1, dtype=torch.int64)
    for i, ln in enumerate(lengths):
        offsets[i + 1] = offsets[i] + ln
    q = torch.empty(B, w.n_layers, S, Hq, d, dtype=w.dtype)
    k = torch.empty(w.n_layers, int(offsets[-1]) + B * L, Hkv, d, dtype=w.dtype)
    for i, (s0, ln) in enumerate(zip(starts, lengths)):
        gw = torch.Generator("cpu").manual_seed(w.seed + 7919 * (i + 1))
        kb = int(offsets[i]) + i * L
        for layer in range(w.n_layers):
            qq = torch.randn(S, Hq, d, generator=gw, dtype=torch.float32)
            kk = torch.randn(ln + L, Hkv, d, generator=gw, dtype=torch.float32)
            for grp in range(Hkv):
                v = qq[:, grp * G:(grp + 1) * G, :].reshape(-1, d).mean(dim=0)
                u = v / v.norm()
                for c, st in zip(spans, strengths):
                    a, b = max(32 * c, s0), min(32 * c + 32, s0 + ln)
                    if a < b:
                        kk[a - s0:b - s0, grp, :] += float(st) * u
            q[i, layer].copy_(qq.to(q.dtype))
            k[layer, kb:kb + ln + L].copy_(kk.to(k.dtype))
    batch = Inputs(w, list(lengths), offsets, q, k, torch.zeros(int(offsets[-1]), dtype=torch.int32),
                   [[] for _ in range(B)], [[] for _ in range(B)])
    return WindowInputs(w, n, list(starts), batch, ids, spans, strengths)
