"""Benchmark of the token-importance path on one MI355X.

One step = the whole path on one batch: sp_score_attention, sp_pool_chunk,
sp_select_chunks and sp_gather_kept, from Q/K/token ids resident in HBM to
the kept-token list. Prints one JSON line with whole-path throughput in
prompt tokens per second, the scoring kernel's achieved HBM bandwidth against
the 8 TB/s peak, and the CPU oracle timed on the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--algo auto|two_pass|stream]
    python bench.py --copy-calibration   # plain device copies of known size (for counters)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prompt tokens scored+selected/s at N=131072; % of HBM bandwidth roofline"
HBM_PEAK_GBS = 8000.0
# HBM traffic of the scoring kernel from hardware counters (two rocprofv3 --pmc
# passes, FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size). Valid
# only for the kernel sources it was measured on.
TRAFFIC_FILES = os.path.join(ROOT, "profiles", "k_stream_*_traffic.md")
KERNEL_SOURCES = ("draft_attention_token_amd/csrc/score_stream.hip",
                  "draft_attention_token_amd/csrc/score_common.h")
COPY_BYTES = 1 << 30


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """Bytes per scoring launch from the committed counter summary, or None if
    it is missing, covers another workload or older kernel sources."""
    for path in sorted(glob.glob(TRAFFIC_FILES)):
        with open(path) as fh:
            fields = dict(re.findall(r"^- (\w+): (\S+)$", fh.read(), re.M))
        if fields.get("workload") != workload or fields.get("source_hash") != kernel_source_hash():
            continue
        try:
            return float(fields["bytes_per_launch"])
        except (KeyError, ValueError):
            return None
    return None


def copy_calibration():
    """Plain device-to-device copies of COPY_BYTES (reads and writes that many
    bytes each): the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)


def achievable_read_gbs(dev):
    """A plain streaming read of 1 GiB (draft_attention_token_amd/bench/
    read_peak.hip, built into libspbench.so), best launch shape of a few,
    median of 9 timed passes each: the read bandwidth this part reaches in
    practice, next to the 8 TB/s peak. Returns (GB/s, blocks per CU)."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "draft_attention_token_amd", "libspbench.so")
    lib = ctypes.CDLL(path)
    lib.spbench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.spbench_read.restype = ctypes.c_int
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    best = (0.0, 0)
    for per_cu in (1, 2, 4, 8):
        def once():
            rc = lib.spbench_read(ctypes.c_void_p(x.data_ptr()), COPY_BYTES,
                                  ctypes.c_void_p(flag.data_ptr()), per_cu,
                                  ctypes.c_void_p(st.cuda_stream))
            assert rc == 0, rc
        for _ in range(3):
            once()
        times = []
        for _ in range(9):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            once()
            b.record(st)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        times.sort()
        gbs = COPY_BYTES / times[len(times) // 2] / 1e9
        best = max(best, (gbs, per_cu))
    del x
    return best


def achievable_korder_gbs(dev, k):
    """The K cache itself read in the scoring kernel's order, with no compute
    and no exchange (read_peak.hip's k_read_heads: problem by problem, the
    KV head's segment of every key row, 32- or 64-key groups dealt to the
    blocks round-robin), best of a few grid sizes, median of 9 timed passes
    each: what this access pattern reaches on this part. Returns (GB/s,
    blocks)."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "draft_attention_token_amd", "libspbench.so")
    lib = ctypes.CDLL(path)
    lib.spbench_read_heads.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.spbench_read_heads.restype = ctypes.c_int
    n_layers, n_keys, hkv, d = k.shape
    nbytes = k.numel() * k.element_size()
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = (0.0, 0)
    for blocks in (cus - 8, cus, 2 * cus):
        def once():
            rc = lib.spbench_read_heads(ctypes.c_void_p(k.data_ptr()), n_layers, n_keys, hkv,
                                        d * k.element_size(), ctypes.c_void_p(flag.data_ptr()),
                                        blocks, ctypes.c_void_p(st.cuda_stream))
            assert rc == 0, rc
        for _ in range(3):
            once()
        times = []
        for _ in range(9):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            once()
            b.record(st)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        times.sort()
        best = max(best, (nbytes / times[len(times) // 2] / 1e9, blocks))
    return best


def score_algorithmic_bytes(inp) -> int:
    """Bytes the scoring stage must move at least once: K and Q read, the
    fp32 importance written."""
    w = inp.workload
    return inp.k.numel() * inp.k.element_size() + inp.q.numel() * inp.q.element_size() + \
        4 * int(inp.offsets[-1])


def host_cpu():
    """The host's CPU model (/proc/cpuinfo) and logical CPU count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def cpu_baseline(inp, mode, param):
    """The oracle as it stands, timed on the host: the whole workload on every
    thread OpenMP gives it (median of 3), and on one core a bounded sample,
    layer 0 alone (1/layers of the scoring work; pooling, selection and
    compaction are a small fraction of it), median of 3, scaled to the whole
    workload."""
    import numpy as np

    import oracle
    w = inp.workload
    threads = oracle.max_threads()
    toks = int(inp.offsets[-1])
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.pipeline(inp, mode, param, nthreads=threads)
        runs.append(time.perf_counter() - t0)
    dt = _median(runs)
    row_pool = w.pool_window if w.pool_before_max else 1
    q1 = np.ascontiguousarray(inp.q[:, :1].float().numpy())
    k1 = inp.k[:1]
    ks1 = None if inp.k_scales is None else inp.k_scales[:1]
    runs1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.importance(inp.offsets.numpy(), q1, k1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim,
                          w.n_lookahead, inp.scale, 1, k_scales=ks1, prefill_row=w.prefill_row,
                          row_pool=row_pool)
        runs1.append(time.perf_counter() - t0)
    dt1 = _median(runs1) * w.n_layers
    model, nproc = host_cpu()
    return {"value": toks / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload {w.name}: {len(inp.lengths)} prompt(s), {toks} tokens, all "
                      f"{w.n_layers} layers; fp64 C loops, OpenMP over (prompt, step, layer); "
                      f"median of 3 runs: {dt:.2f} s",
            "seconds": dt, "runs": runs, "cpu_model": model, "nproc": nproc,
            "one_core": {"value": toks / dt1, "unit": "tokens/s", "cores": 1,
                         "sample": f"importance of layer 0 alone, median of 3 runs "
                                   f"({_median(runs1):.2f} s), times {w.n_layers} layers",
                         "seconds_scaled": dt1}}


def cpu_baseline_tool(win_inp):
    """The oracle as it stands on the standalone tool's path (its own window
    plan), on every host thread OpenMP gives it, median of 3."""
    import oracle
    w = win_inp.workload
    plan = oracle.window_plan(win_inp.n_tokens, w.window, w.stride)
    threads = oracle.max_threads()
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.tool_pipeline(win_inp, plan, nthreads=threads)
        runs.append(time.perf_counter() - t0)
    dt = _median(runs)
    toks = win_inp.n_tokens
    model, nproc = host_cpu()
    return {"value": toks / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload {w.name}: {toks} tokens in {len(plan)} windows; fp64 C "
                      f"loops, OpenMP over (window, step, layer); median of 3 runs: {dt:.2f} s",
            "seconds": dt, "runs": runs, "cpu_model": model, "nproc": nproc}


def scoring_kernels(pipe, fp8k, w):
    """The scoring kernels a call runs, as the library reports them."""
    plan = __import__("draft_attention_token_amd.specprefill", fromlist=["score_plan"]).score_plan(
        pipe.adesc, pipe.batch)
    launches = f", {plan.n_launches} launches" if plan.n_launches > 1 else ""
    if plan.kernel == "stream":
        return f"k_stream<{w.head_dim}, fp8 K={fp8k}> (sp_score_attention{launches})"
    last = "k_score_pooled" if w.pool_before_max else "k_score"
    return f"k_stats + k_lse + {last} (sp_score_attention{launches})"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n128k_bf16")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--mode", default=None, help="top_p or mass (default: the workload's)")
    ap.add_argument("--param", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(prompts of a batch are independent; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from draft_attention_token_amd import specprefill as sp

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    mode, param = (args.mode, args.param) if args.mode else w.select
    log(f"generating {w.name}")
    tool = w.window > 0
    if tool:
        # The standalone tool: the prompt's windows (planned by the library)
        # are scored as one batch, then stitched and selected.
        n_tok = int(w.lengths[0])
        starts, lengths, _ = sp.window_plan(n_tok, w.window, w.stride)
        win_inp = workloads.make_window_inputs(w, starts, lengths)
        inp = win_inp.batch
        ids = win_inp.token_ids.to(dev)
        tokens = n_tok
        pipe = sp.ToolPipeline(n_tok, w.window, w.stride, w.n_layers, w.n_q_heads, w.n_kv_heads,
                               w.head_dim, w.n_lookahead, w.dtype, dev, C=w.chunk_size,
                               W=w.pool_window, normalize=w.normalize, boost=w.boost,
                               keep_pct=w.keep_pct, min_tokens=w.min_tokens,
                               max_keep=w.max_keep, prefill_row=w.prefill_row, algo=args.algo)
        mode, param = "legacy", w.keep_pct
    else:
        inp = workloads.make_inputs(w)
        ids = inp.token_ids.to(dev)
        tokens = int(inp.offsets[-1])
        pipe = sp.Pipeline(inp.offsets, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim,
                           w.n_lookahead, w.dtype, dev, W=w.pool_window, C=w.chunk_size,
                           normalize=w.normalize, boost=w.boost, mode=mode, param=param,
                           algo=args.algo, k_dtype=inp.k.dtype, k_scales=inp.k_scales,
                           prefill_row=w.prefill_row, pool_before_max=w.pool_before_max)
    q, k = inp.q.to(dev), inp.k.to(dev)
    torch.cuda.synchronize()
    fp8k = inp.k.dtype == torch.float8_e4m3fn
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        pipe.run(q, k, ids)
    torch.cuda.synchronize()

    # Whole path: K steps between two events on the stream the calls use.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t_host = time.perf_counter()
    for _ in range(args.steps):
        pipe.run(q, k, ids)
    e1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"whole path {ms_step * 1e3:.1f} us/step (host clock {t_host / args.steps * 1e6:.1f} us)")
    # The same steps one by one, each between its own events: the median.
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in per:
        a.record(stream)
        pipe.run(q, k, ids)
        b.record(stream)
    torch.cuda.synchronize()
    ms_step_median = sorted(a.elapsed_time(b) for a, b in per)[args.steps // 2]
    log(f"whole path median of {args.steps} single steps: {ms_step_median * 1e3:.1f} us")

    # Scoring stage alone, same stream, same inputs: one pair of events around
    # each launch (the scoring call is one kernel launch per batch of up to
    # 256 blocks' worth of prompts), averaged.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        pipe.run_score(q, k)
        b.record(stream)
    torch.cuda.synchronize()
    assert pipe.score_status() == 0, "scoring kernel reported a timed-out wait"
    ms_score = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    # The stages after scoring alone, the same way.
    for a, b in ev:
        a.record(stream)
        pipe.run_post(ids)
        b.record(stream)
    torch.cuda.synchronize()
    ms_post = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    if tool:
        post_form = "sp_stitch_windows + sp_pool_chunk + sp_select_legacy"
    else:
        assert pipe.post_status() == 0, "post-scoring launch reported a timed-out wait"
        form, tb = sp.post_form(pipe.pdesc, pipe.batch)
        post_form = {"die": f"sp_pool_select_gather: one die-local launch, {tb}-token ranges",
                     "grid": f"sp_pool_select_gather: one launch, {tb}-token blocks",
                     "separate": "sp_pool_select_gather: separate pool, select and gather kernels"}[form]
    log(f"after scoring: {ms_post * 1e3:.1f} us ({post_form})")
    alg_bytes = score_algorithmic_bytes(inp)
    achieved = alg_bytes / (ms_score * 1e-3) / 1e9
    log(f"scoring {ms_score * 1e3:.1f} us per launch -> {achieved:.0f} GB/s algorithmic")
    traffic = measured_traffic(w.name)
    read_gbs, read_shape = achievable_read_gbs(dev)
    log(f"plain 1 GiB streaming read: {read_gbs:.0f} GB/s ({read_shape} blocks per CU)")
    korder_gbs, korder_blocks = achievable_korder_gbs(dev, k)
    log(f"K read in the scoring order: {korder_gbs:.0f} GB/s ({korder_blocks} blocks)")

    kept = int(pipe.kept_offsets[-1])
    kernel_name = scoring_kernels(pipe, fp8k, w)
    if tool:
        kernel_name += " on the window batch"
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_step_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "prompts": len(inp.lengths), "prompt_tokens": tokens,
                   "lookahead": w.n_lookahead, "layers": w.n_layers, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "pool_window": w.pool_window,
                   "chunk": w.chunk_size, "normalize": w.normalize, "boost": w.boost,
                   "select": f"{mode} {param}", "score_algo": args.algo, "kept_tokens": kept,
                   "k_cache": "fp8 e4m3 codes, fp32 scale per (layer, KV head)" if fp8k
                   else "same type as Q",
                   "prefill_row": w.prefill_row, "pool_before_max": w.pool_before_max,
                   **({"window": w.window, "stride": w.stride, "windows": len(inp.lengths),
                       "window_tokens": int(inp.offsets[-1]), "max_keep": w.max_keep}
                      if tool else {})},
        "stages": {"score_us": ms_score * 1e3, "post_us": ms_post * 1e3, "post": post_form},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_name,
                     "launch_us": ms_score * 1e3,
                     "algorithmic_bytes": alg_bytes,
                     "achievable": {"read": read_gbs, "frac": achieved / read_gbs,
                                    "kernel": f"k_read, plain streaming read of 1 GiB, "
                                              f"{read_shape} x 512 threads per CU",
                                    "k_order_read": korder_gbs,
                                    "k_order_frac": achieved / korder_gbs,
                                    "k_order_kernel": f"k_read_heads, the K cache read problem by "
                                                      f"problem as the scoring kernel reads it, "
                                                      f"no compute, {korder_blocks} x 512 "
                                                      f"threads"}},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = (cpu_baseline_tool(win_inp) if tool else
                                  cpu_baseline(inp, mode, param))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
