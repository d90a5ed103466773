"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Small shapes cover several tiles, ragged tails, every supported dtype /
head size / group size, both scoring kernels and the batch edge cases; the
named workloads run at their full sizes (the ragged batch compares every
prompt of every scoring launch end to end).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from draft_attention_token_amd import specprefill as sp

from parity import KEY_TOL, SUM_TOL, assert_scores_close, check_prompt, excused_chunks

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    sp.lib()


def run_gpu(inp, mode, param, algo="auto"):
    w = inp.workload
    print(f"[gpu] {w.name} lengths={inp.lengths[:4]}{'...' if len(inp.lengths) > 4 else ''} "
          f"mode={mode} p={param} algo={algo}", flush=True)
    pipe = sp.Pipeline(inp.offsets, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim,
                       w.n_lookahead, w.dtype, DEV, W=w.pool_window, C=w.chunk_size,
                       normalize=w.normalize, boost=w.boost, mode=mode, param=param, algo=algo,
                       k_dtype=inp.k.dtype, k_scales=inp.k_scales, prefill_row=w.prefill_row,
                       pool_before_max=w.pool_before_max)
    q, k, ids = inp.q.to(DEV), inp.k.to(DEV), inp.token_ids.to(DEV)
    pipe.run(q, k, ids)
    torch.cuda.synchronize()
    assert pipe.score_status() == 0, "scoring kernel reported a timed-out wait"
    return pipe


def per_prompt(pipe, inp):
    off = inp.offsets.numpy()
    C = inp.workload.chunk_size
    coff = np.concatenate([[0], np.cumsum([(n + C - 1) // C for n in inp.lengths])])
    koff = pipe.kept_offsets.cpu().numpy()
    cs, keep = pipe.chunk_scores.cpu().numpy(), pipe.keep.cpu().numpy()
    kid, kpos = pipe.kept_ids.cpu().numpy(), pipe.kept_pos.cpu().numpy()
    imp = pipe.importance.cpu().numpy()
    ts = pipe.token_scores.cpu().numpy()
    out = []
    for b in range(len(inp.lengths)):
        out.append(dict(imp=imp[off[b]:off[b + 1]], token_scores=ts[off[b]:off[b + 1]],
                        chunk_scores=cs[coff[b]:coff[b + 1]], keep=keep[coff[b]:coff[b + 1]],
                        kept_ids=kid[koff[b]:koff[b + 1]], kept_pos=kpos[koff[b]:koff[b + 1]]))
    assert koff[0] == 0 and np.all(np.diff(koff) > 0)
    return out


def compare(inp, pipe, mode, param, prompts=None, ora=None):
    w = inp.workload
    if prompts is None:
        prompts = range(len(inp.lengths))
    if ora is None:
        ora = oracle.pipeline(inp, mode, param)
    gp = per_prompt(pipe, inp)
    ids = inp.token_ids.numpy()
    off = inp.offsets.numpy()
    excused = 0
    for b in prompts:
        assert_scores_close(gp[b]["imp"], ora["imp"][off[b]:off[b + 1]], f"importance, prompt {b}")
        assert_scores_close(gp[b]["token_scores"], ora["token_scores"][b], f"token scores, prompt {b}")
        excused += check_prompt(gp[b], ora, b, mode, param, w.chunk_size, ids[off[b]:off[b + 1]])
    n_kept = pipe.n_kept.cpu().numpy()
    for b in prompts:
        assert n_kept[b] == gp[b]["keep"].sum()
    return excused, gp


SMALL = [
    # (name, base workload, overrides)
    ("fp32_d64_g4", "n800_fp32", dict(lengths=(333,))),
    ("fp32_d64_one_token", "n800_fp32", dict(lengths=(1,))),
    ("fp32_d64_ragged", "n800_fp32", dict(lengths=(31, 32, 33, 97))),
    ("fp32_d128_g2_l3", "n800_fp32", dict(lengths=(250, 71), head_dim=128, n_q_heads=4,
                                           n_kv_heads=2, n_lookahead=3)),
    ("bf16_d128_g4", "n3212_bf16", dict(lengths=(1000,))),
    ("bf16_d128_ragged", "n3212_bf16", dict(lengths=(65, 1, 640, 129))),
    ("bf16_d64_g8_l4", "n3212_bf16", dict(lengths=(500,), head_dim=64, n_q_heads=16,
                                          n_kv_heads=2, n_lookahead=4)),
    ("bf16_d128_g1_l1", "n3212_bf16", dict(lengths=(300, 45), n_q_heads=4, n_kv_heads=4,
                                           n_lookahead=1)),
    ("bf16_d128_g32_l1", "n3212_bf16", dict(lengths=(200,), n_q_heads=32, n_kv_heads=1,
                                            n_lookahead=1, n_layers=2)),
    ("bf16_no_norm", "n3212_bf16", dict(lengths=(800,), normalize=False, boost=False)),
    # The prefill's last row as step 0.
    ("prerow_bf16_d128_g4_l7", "n3212_prerow_bf16", dict(lengths=(1000,))),
    ("prerow_bf16_ragged", "n3212_prerow_bf16", dict(lengths=(65, 1, 640, 129, 2))),
    ("prerow_fp32_d64_alone", "n800_fp32", dict(lengths=(333, 2, 1), n_lookahead=0,
                                                 prefill_row=True)),
    ("prerow_bf16_d64_g8_l3", "n3212_bf16", dict(lengths=(500,), head_dim=64, n_q_heads=16,
                                                 n_kv_heads=2, n_lookahead=3, prefill_row=True)),
    # Pool-before-max (two-pass kernels whatever the algo asks).
    ("poolmax_bf16_d128_g4", "n3212_poolmax_bf16", dict(lengths=(1000,))),
    ("poolmax_bf16_ragged", "n3212_poolmax_bf16", dict(lengths=(65, 1, 640, 129, 7, 13))),
    ("poolmax_fp32_d64_w33", "n800_fp32", dict(lengths=(333, 40), pool_before_max=True,
                                                pool_window=33)),
    # Fewer problems than waves per tile (idle waves in a round).
    ("poolmax_bf16_one_problem", "n3212_poolmax_bf16", dict(lengths=(700, 33), n_layers=1,
                                                            n_q_heads=4, n_kv_heads=1)),
    ("poolmax_bf16_three_problems", "n3212_poolmax_bf16", dict(lengths=(300,), n_layers=3,
                                                               n_q_heads=4, n_kv_heads=1)),
    # Three heads per group: the head max through LDS atomics, not lane shuffles.
    ("poolmax_bf16_g3", "n3212_poolmax_bf16", dict(lengths=(400, 21), n_q_heads=6, n_kv_heads=2,
                                                   n_lookahead=4)),
    ("bf16_g3_two_pass", "n3212_bf16", dict(lengths=(400, 21), n_q_heads=6, n_kv_heads=2,
                                            n_lookahead=4)),
    ("poolmax_bf16_d64_g8_w3_prerow", "n3212_bf16", dict(lengths=(500, 31), head_dim=64,
                                                         n_q_heads=16, n_kv_heads=2, n_lookahead=3,
                                                         prefill_row=True, pool_before_max=True,
                                                         pool_window=3)),
]


def stream_runs(w):
    """Whether the single-pass kernel takes the workload's shape: bf16 Q, no
    pooling before the max, 2^k heads per group."""
    g = w.n_q_heads // w.n_kv_heads
    return w.dtype == torch.bfloat16 and not w.pool_before_max and g & (g - 1) == 0


# AUTO scores batches this short with the two-pass kernels, so the single-pass
# kernel is asked for by name too.
@pytest.mark.parametrize("algo", ["two_pass", "auto", "stream"])
@pytest.mark.parametrize("name, base, kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(name, base, kw, algo):
    w = workloads.small_workload(base, seed=500 + len(name), n_spans=2, **kw)
    if algo == "stream" and not stream_runs(w):
        pytest.skip("shape taken by the two-pass kernels only")
    inp = workloads.make_inputs(w)
    for mode, param in (("top_p", 0.3), ("mass", 0.85)):
        pipe = run_gpu(inp, mode, param, algo)
        compare(inp, pipe, mode, param)


@pytest.mark.parametrize("algo", ["auto", "stream"])
@pytest.mark.parametrize("name", ["n800_fp32", "n3212_bf16", "n3212_prerow_bf16",
                                  "n3212_poolmax_bf16"])
def test_named_small_workloads(name, algo):
    w = workloads.WORKLOADS[name]
    if algo == "stream" and not stream_runs(w):
        pytest.skip("shape taken by the two-pass kernels only")
    inp = workloads.make_inputs(w)
    for mode, param in (w.select,) + tuple(w.also_select):
        pipe = run_gpu(inp, mode, param, algo)
        compare(inp, pipe, mode, param)
        keep = pipe.keep.cpu().numpy()
        for c in inp.spans[0]:
            assert keep[c] == 1, f"planted chunk {c} dropped"


def test_all_zero_queries_give_equal_chunk_scores():
    w = workloads.small_workload("n3212_bf16", lengths=(900,), normalize=False, boost=False)
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    pipe = run_gpu(inp, "top_p", 0.3)
    imp = pipe.importance.cpu().numpy().astype(np.float64)
    want = sum(1.0 / (900 + j + 1) for j in range(8)) / 8
    np.testing.assert_allclose(imp, want, rtol=1e-6)
    cs = pipe.chunk_scores.cpu().numpy()
    np.testing.assert_allclose(cs, cs[0], rtol=1e-6)


@pytest.mark.parametrize("algo", ["auto", "stream"])
def test_flat_scores_normalise_to_one_then_boost(algo):
    """All-zero queries give every prompt token the same importance: the
    scores carry no signal, so normalisation makes each 1.0 before the boosts
    (first 64 tokens x1.5, last 128 x1.3), as in the oracle."""
    w = workloads.small_workload("n3212_bf16", lengths=(900,), normalize=True, boost=True)
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    want = np.ones(900)
    want[:64] *= 1.5
    want[-128:] *= 1.3
    for mode, param in (("top_p", 0.3), ("mass", 0.85)):
        pipe = run_gpu(inp, mode, param, algo)
        np.testing.assert_allclose(pipe.token_scores.cpu().numpy(), want, rtol=1e-6)
        compare(inp, pipe, mode, param, ora=oracle.pipeline(inp, mode, param))


def test_timed_out_call_leaves_the_workspace_usable(monkeypatch):
    """A zero wait budget (SP_SCORE_WAIT_US=0, read by the host at launch)
    makes every cross-block wait of the single pass give up at once: the
    kernels still drain, the call reports the time-out and a checked
    pipeline raises. The next call on the same workspace with the normal
    budget succeeds and matches a call on a fresh workspace, bit for bit:
    slots carry the tag of the call that wrote them, so nothing the failed
    call left behind is taken for a result."""
    w = workloads.small_workload("n32k_bf16", lengths=(20000,), n_spans=4)
    inp = workloads.make_inputs(w)
    q, k = inp.q.to(DEV), inp.k.to(DEV)
    batch = sp.Batch(inp.offsets)
    desc = sp.attn_desc(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_lookahead, w.dtype,
                        algo="stream")
    nbytes = sp.score_workspace_bytes(desc, batch)
    ws, fresh = sp._ws(nbytes, DEV), sp._ws(nbytes, DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)

    def call(wsx):
        out = torch.full((batch.total,), float("nan"), dtype=torch.float32, device=DEV)
        rc = sp.lib().sp_score_attention(ctypes.byref(desc), batch.ref(),
                                         ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(wsx.data_ptr()), wsx.numel(), st)
        assert rc == sp.SP_OK, sp.status_string(rc)
        torch.cuda.synchronize()
        return out

    monkeypatch.setenv("SP_SCORE_WAIT_US", "0")
    print("[gpu] scoring with a zero wait budget", flush=True)
    call(ws)
    assert sp.score_status(ws) == 1
    pipe = sp.Pipeline(inp.offsets, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim,
                       w.n_lookahead, w.dtype, DEV, algo="stream")
    with pytest.raises(sp.SpError):
        pipe.run(q, k, inp.token_ids.to(DEV), check=True)
    monkeypatch.delenv("SP_SCORE_WAIT_US")
    again = call(ws)
    assert sp.score_status(ws) == 0
    ref = call(fresh)
    assert sp.score_status(fresh) == 0
    assert torch.equal(again, ref)
    pipe.run(q, k, inp.token_ids.to(DEV), check=True)


@pytest.mark.parametrize("algo", ["auto", "stream"])
def test_results_are_bitwise_deterministic(algo):
    w = workloads.small_workload("n3212_bf16", lengths=(2000, 3000), seed=9)
    inp = workloads.make_inputs(w)
    a = run_gpu(inp, "mass", 0.85, algo)
    imp1, cs1 = a.importance.clone(), a.chunk_scores.clone()
    ids1 = a.kept_ids.clone()
    b = run_gpu(inp, "mass", 0.85, algo)
    assert torch.equal(imp1, b.importance)
    assert torch.equal(cs1, b.chunk_scores)
    n = int(b.kept_offsets[-1])
    assert torch.equal(ids1[:n], b.kept_ids[:n])


def test_score_workspace_reused_across_batches_and_algorithms():
    """One zero-filled scoring workspace serves calls with different batches and
    both kernels in any order: each call's cross-block slots are tagged with the
    call, so what an earlier call left behind is never taken for a result."""
    w = workloads.small_workload("n3212_bf16", lengths=(2500, 700), seed=33)
    base = workloads.make_inputs(w)
    other = workloads.make_inputs(w, lengths=(4100,))
    big = max(sp.score_workspace_bytes(sp.attn_desc(w.n_layers, w.n_q_heads, w.n_kv_heads,
                                                    w.head_dim, w.n_lookahead, w.dtype), sp.Batch(x.offsets))
              for x in (base, other))
    ws = torch.zeros(big, dtype=torch.uint8, device=DEV)

    def score(inp, algo, ws_):
        return sp.sp_score_attention(inp.q.to(DEV), inp.k.to(DEV), inp.offsets, w.n_layers,
                                     w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_lookahead,
                                     algo=algo, ws=ws_)

    fresh = {}
    for name, inp in (("base", base), ("other", other)):
        for algo in ("stream", "two_pass"):
            fresh[name, algo] = score(inp, algo, None).cpu()
    order = [("base", "stream"), ("other", "stream"), ("base", "two_pass"), ("base", "stream"),
             ("other", "two_pass"), ("other", "stream"), ("base", "stream")]
    for name, algo in order:
        got = score(base if name == "base" else other, algo, ws)
        torch.cuda.synchronize()
        assert sp.score_status(ws) == 0
        assert torch.equal(got.cpu(), fresh[name, algo]), (name, algo)
    ora = oracle.importance(base.offsets.numpy(), base.q, base.k, w.n_layers, w.n_q_heads,
                            w.n_kv_heads, w.head_dim, w.n_lookahead, base.scale)
    assert_scores_close(fresh["base", "stream"].numpy(), ora, "importance")


SELECT_SCORE_KINDS = ["uniform", "ties", "equal", "zero", "spiky"]


def _select_scores(kind, nc, rng):
    if kind == "uniform":
        return rng.random(nc).astype(np.float32)
    if kind == "ties":
        return rng.choice(np.array([0.0, 0.25, 0.5, 1.0], dtype=np.float32), nc)
    if kind == "equal":
        return np.full(nc, 0.7, dtype=np.float32)
    if kind == "zero":
        return np.zeros(nc, dtype=np.float32)
    x = (rng.random(nc) ** 8).astype(np.float32)        # most mass in a few chunks
    x[rng.integers(0, nc, 3)] = 50.0
    return x


@pytest.mark.parametrize("kind", SELECT_SCORE_KINDS)
@pytest.mark.parametrize("mode, params", [("top_p", (0.01, 0.15, 0.5, 1.0)),
                                          ("mass", (0.01, 0.5, 0.85, 1.0))])
def test_select_chunks_edge_cases(kind, mode, params):
    """The selection kernel alone on constructed chunk scores: ties, constant
    and all-zero prompts, a few dominant chunks, 1 to 16384 chunks per prompt,
    several prompts per batch; exact against the oracle's rule."""
    rng = np.random.default_rng(7)
    ncs = [1, 2, 3, 33, 1000, 4096, 16384]
    offsets = np.concatenate([[0], np.cumsum([32 * n for n in ncs])]).astype(np.int64)
    batch = sp.Batch(offsets)
    scores = [_select_scores(kind, n, rng) for n in ncs]
    cs = torch.from_numpy(np.concatenate(scores)).to(DEV)
    coff = np.concatenate([[0], np.cumsum(ncs)])
    for param in params:
        keep, cnt = sp.sp_select_chunks(cs, batch, 32, mode, param)
        keep, cnt = keep.cpu().numpy(), cnt.cpu().numpy()
        for bi, n in enumerate(ncs):
            got = keep[coff[bi]:coff[bi + 1]]
            sc64 = scores[bi].astype(np.float64)
            want = oracle.select(sc64, mode, param)
            diff = np.flatnonzero(got != want)
            if diff.size:
                # Only where the kernel's fixed-point order and sums may
                # legitimately differ from fp64 (see tests/parity.py).
                assert kind in ("uniform", "spiky"), (kind, mode, param, n, diff[:10])
                ex = excused_chunks(sc64, want, mode, param, cutoff_tol=KEY_TOL * sc64.max(),
                                    mass_tol=SUM_TOL)
                bad = [int(i) for i in diff if int(i) not in ex]
                assert not bad, (kind, mode, param, n, bad[:10])
            assert cnt[bi] == int(got.sum())


def test_pool_select_gather_stages_on_oracle_importance():
    """Stages after scoring, fed the oracle's importance (rounded to fp32)."""
    w = workloads.small_workload("n3212_bf16", lengths=(3212, 100, 5000), seed=21)
    inp = workloads.make_inputs(w)
    imp = oracle.importance(inp.offsets.numpy(), inp.q, inp.k, w.n_layers, w.n_q_heads,
                            w.n_kv_heads, w.head_dim, w.n_lookahead, inp.scale)
    imp32 = imp.astype(np.float32)
    ora = oracle.pipeline(inp, "top_p", 0.3, imp=imp32.astype(np.float64))
    batch = sp.Batch(inp.offsets)
    ts, cs = sp.sp_pool_chunk(torch.from_numpy(imp32).to(DEV), batch)
    keep, cnt = sp.sp_select_chunks(cs, batch, 32, "top_p", 0.3)
    kid, kpos, koff = sp.sp_gather_kept(keep, inp.token_ids.to(DEV), batch, 32)
    torch.cuda.synchronize()
    off = inp.offsets.numpy()
    ts, cs, keep = ts.cpu().numpy(), cs.cpu().numpy(), keep.cpu().numpy()
    koff, kid, kpos = koff.cpu().numpy(), kid.cpu().numpy(), kpos.cpu().numpy()
    c0 = 0
    for b, n in enumerate(inp.lengths):
        nc = (n + 31) // 32
        assert_scores_close(ts[off[b]:off[b + 1]], ora["token_scores"][b], f"token scores {b}")
        assert_scores_close(cs[c0:c0 + nc], ora["chunk_scores"][b], f"chunk scores {b}")
        gpu = dict(chunk_scores=cs[c0:c0 + nc], keep=keep[c0:c0 + nc],
                   kept_ids=kid[koff[b]:koff[b + 1]], kept_pos=kpos[koff[b]:koff[b + 1]])
        check_prompt(gpu, ora, b, "top_p", 0.3, 32, inp.token_ids.numpy()[off[b]:off[b + 1]])
        c0 += nc


FP8K_SMALL = [
    ("fp8k_d128_g4", "n3212_fp8k", dict(lengths=(1000,))),
    ("fp8k_d128_ragged", "n3212_fp8k", dict(lengths=(65, 1, 640, 129))),
    ("fp8k_d64_g8_l4", "n3212_fp8k", dict(lengths=(500,), head_dim=64, n_q_heads=16,
                                          n_kv_heads=2, n_lookahead=4)),
    ("fp8k_d128_g1_l1", "n3212_fp8k", dict(lengths=(300, 45), n_q_heads=4, n_kv_heads=4,
                                           n_lookahead=1)),
    ("fp8k_prerow_l7", "n3212_fp8k", dict(lengths=(700, 33), n_lookahead=7, prefill_row=True)),
]


@pytest.mark.parametrize("name, base, kw", FP8K_SMALL, ids=[s[0] for s in FP8K_SMALL])
def test_fp8k_small_shapes(name, base, kw):
    """fp8 e4m3 K codes with per-(layer, KV head) scales, bf16 Q."""
    w = workloads.small_workload(base, seed=700 + len(name), n_spans=2, **kw)
    inp = workloads.make_inputs(w)
    assert inp.k.dtype == torch.float8_e4m3fn and inp.k_scales is not None
    for mode, param in (("top_p", 0.3), ("mass", 0.85)):
        pipe = run_gpu(inp, mode, param)
        compare(inp, pipe, mode, param)


@pytest.mark.parametrize("name", ["n32k_bf16", "n128k_bf16", "n128k_diffuse_bf16", "n128k_fp8k",
                                  "n32k_prerow_bf16", "n128k_poolmax_bf16"])
def test_full_size_single_prompt(name):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    imp = oracle.importance(inp.offsets.numpy(), inp.q, inp.k, w.n_layers, w.n_q_heads,
                            w.n_kv_heads, w.head_dim, w.n_lookahead, inp.scale,
                            k_scales=inp.k_scales, prefill_row=w.prefill_row,
                            row_pool=w.pool_window if w.pool_before_max else 1)
    for mode, param in (w.select,) + tuple(w.also_select):
        pipe = run_gpu(inp, mode, param)
        ora = oracle.pipeline(inp, mode, param, imp=imp)
        excused, _ = compare(inp, pipe, mode, param, ora=ora)
        print(f"[gpu] {name} {mode}: excused differing chunks = {excused}", flush=True)
        keep = pipe.keep.cpu().numpy()
        # Pooling every row before the max dilutes the weakest spans: at top-p
        # 0.15 the oracle itself drops one of strength 0.56 there.
        floor = 1.0 if w.pool_before_max else 0.0
        for c, st in zip(inp.spans[0], inp.strengths[0]):
            assert keep[c] == 1 or st < floor, f"planted chunk {c} dropped"


@pytest.mark.parametrize("name", ["n160k_bf16", "n160k_fp8k"])
def test_single_pass_at_163840_tokens(name):
    """The longest prompt one single-pass launch takes (5121 tiles over 248
    blocks of at most 21): the plan must keep it in one launch of the single
    pass, and its results must match the oracle's."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    desc = sp.attn_desc(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_lookahead, w.dtype,
                        k_dtype=inp.k.dtype, k_scales=inp.k_scales)
    plan = sp.score_plan(desc, sp.Batch(inp.offsets))
    assert plan.kernel == "stream" and plan.n_launches == 1, plan
    imp = oracle.importance(inp.offsets.numpy(), inp.q, inp.k, w.n_layers, w.n_q_heads,
                            w.n_kv_heads, w.head_dim, w.n_lookahead, inp.scale,
                            k_scales=inp.k_scales)
    for mode, param in (w.select,) + tuple(w.also_select):
        pipe = run_gpu(inp, mode, param)
        ora = oracle.pipeline(inp, mode, param, imp=imp)
        excused, _ = compare(inp, pipe, mode, param, ora=ora)
        print(f"[gpu] {name} {mode}: excused differing chunks = {excused}", flush=True)
        keep = pipe.keep.cpu().numpy()
        for c in inp.spans[0]:
            assert keep[c] == 1, f"planted chunk {c} dropped"


@pytest.mark.parametrize("n", [70000, 9000])
def test_fold_lag_forms(n):
    """The single-pass kernel keeps 3, 4 or 7 problems parked, by how many
    tiles its compute waves own: 70000 tokens over 248 blocks give 9 tiles
    per block, at most 2 per wave (4 parked), 9000 tokens 2 per block, at
    most 1 per wave (7 parked); the 128K prompts above own up to 3 (3
    parked)."""
    w = workloads.small_workload("n32k_bf16", lengths=(n,), n_spans=8)
    inp = workloads.make_inputs(w)
    mode, param = w.select
    pipe = run_gpu(inp, mode, param)
    excused, _ = compare(inp, pipe, mode, param)
    print(f"[gpu] lag form n={n}: excused differing chunks = {excused}", flush=True)


def test_ragged_batch_all_prompts():
    """16 prompts of 2K-64K tokens, in the launch configuration the benchmark
    uses: every prompt of every scoring launch is compared with the oracle
    (importance, token and chunk scores, kept chunks, ids and positions), for
    both selection rules on the same scores."""
    w = workloads.WORKLOADS["ragged16_bf16"]
    inp = workloads.make_inputs(w)
    plan = sp.score_plan(sp.attn_desc(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                      w.n_lookahead, w.dtype), sp.Batch(inp.offsets))
    print(f"[gpu] ragged16 plan: kernel={plan.kernel} launches={plan.n_launches} "
          f"prompt_launch={plan.prompt_launch}", flush=True)
    assert plan.kernel == "stream" and plan.n_launches >= 2, plan
    # Every launch holds at least one prompt, and all of them are compared below.
    assert sorted(set(plan.prompt_launch)) == list(range(plan.n_launches))
    imp = oracle.importance(inp.offsets.numpy(), inp.q, inp.k, w.n_layers, w.n_q_heads,
                            w.n_kv_heads, w.head_dim, w.n_lookahead, inp.scale)
    for mode, param in (w.select,) + tuple(w.also_select):
        pipe = run_gpu(inp, mode, param)
        ora = oracle.pipeline(inp, mode, param, imp=imp)
        excused, gp = compare(inp, pipe, mode, param, ora=ora)
        kept = [int(gp[b]["keep"].sum()) for b in range(len(inp.lengths))]
        print(f"[gpu] ragged16 {mode} {param}: kept chunks per prompt {kept}, "
              f"excused differing chunks = {excused}", flush=True)
        for b in range(len(inp.lengths)):
            for c in inp.spans[b]:
                assert gp[b]["keep"][c] == 1, f"prompt {b}: planted chunk {c} dropped"


# ----------------------------------------------------------------------------
# Standalone-tool semantics: windows, stitching, legacy rule, cap
# ----------------------------------------------------------------------------

TOOL_CASES = [
    # (name, base, overrides)
    ("tool4471", "tool4471_bf16", dict()),
    ("tool_fill_and_cap", "tool4471_bf16", dict(lengths=(900,), window=256, stride=128,
                                                keep_pct=0.02, max_keep=70)),
    ("tool_ragged_windows", "tool4471_bf16", dict(lengths=(1337,), window=300, stride=100,
                                                  keep_pct=0.25, chunk_size=16)),
    ("tool_one_window_no_norm", "tool4471_bf16", dict(lengths=(777,), window=2000, stride=1000,
                                                      normalize=False, boost=False, n_lookahead=4)),
    ("tool_128k", "tool128k_bf16", dict()),
]


@pytest.mark.parametrize("name, base, kw", TOOL_CASES, ids=[c[0] for c in TOOL_CASES])
def test_tool_windows_legacy_selection(name, base, kw):
    w = workloads.small_workload(base, **kw)
    n = w.lengths[0]
    starts, lengths, keeps = sp.window_plan(n, w.window, w.stride)
    plan = oracle.window_plan(n, w.window, w.stride)
    assert list(zip(starts, lengths, keeps)) == plan
    wi = workloads.make_window_inputs(w, starts, lengths)
    print(f"[gpu] {name}: n={n} windows={len(plan)} keep={w.keep_pct} cap={w.max_keep}", flush=True)
    pipe = sp.ToolPipeline(n, w.window, w.stride, w.n_layers, w.n_q_heads, w.n_kv_heads,
                           w.head_dim, w.n_lookahead, w.dtype, DEV, C=w.chunk_size,
                           W=w.pool_window, normalize=w.normalize, boost=w.boost,
                           keep_pct=w.keep_pct, min_tokens=w.min_tokens, max_keep=w.max_keep,
                           prefill_row=w.prefill_row)
    ids = wi.token_ids.to(DEV)
    pipe.run(wi.batch.q.to(DEV), wi.batch.k.to(DEV), ids)
    torch.cuda.synchronize()
    assert pipe.score_status() == 0
    ora = oracle.tool_pipeline(wi, plan)
    assert_scores_close(pipe.importance.cpu().numpy(), ora["imp"], "window importance")
    assert_scores_close(pipe.scores.cpu().numpy(), ora["scores"], "stitched scores")
    assert_scores_close(pipe.token_scores.cpu().numpy(), ora["token_scores"], "token scores")
    cs = pipe.chunk_scores.cpu().numpy()
    assert_scores_close(cs, ora["chunk_scores"], "chunk scores")
    off = pipe.kept_offsets.cpu().numpy()
    got_pos = pipe.kept_pos.cpu().numpy()[off[0]:off[1]]
    got_ids = pipe.kept_ids.cpu().numpy()[off[0]:off[1]]
    # The rule and the cap, exactly, on the GPU's own chunk scores.
    own = oracle.thin(oracle.select_legacy_from_means(cs, n, w.chunk_size, w.keep_pct,
                                                      w.min_tokens), w.max_keep)
    np.testing.assert_array_equal(got_pos, own)
    np.testing.assert_array_equal(got_ids, wi.token_ids.numpy()[own])
    # Against the oracle's own scores: identical unless a chunk mean sits
    # within 1e-5 of the oracle's threshold.
    means = np.float32(ora["chunk_scores"])
    nc = means.size
    kc = oracle.legacy_keep_count(nc, w.keep_pct)
    th = np.sort(means)[::-1][kc - 1]
    near = np.abs(means.astype(np.float64) - th) <= 1e-5
    if near.sum() <= 1:                                   # only the threshold chunk itself
        np.testing.assert_array_equal(got_pos, ora["final"])
        np.testing.assert_array_equal(got_ids, ora["final_ids"])
    else:
        print(f"[gpu] {name}: {int(near.sum()) - 1} chunk(s) excused near the threshold", flush=True)
    if ora["kept"].size <= w.max_keep and w.keep_pct >= 0.25:
        for c in wi.spans:                                # planted spans survive an uncapped rule
            assert np.isin(np.arange(32 * c, 32 * c + 32), got_pos).all(), c


@pytest.mark.parametrize("C, keep, min_tok, max_keep", [(32, 0.3, 128, 2000), (1, 0.05, 4, 5),
                                                         (16, 0.01, 10 ** 6, 70), (3, 0.9, 0, 1),
                                                         (32, 1.0, 128, 100)])
def test_select_legacy_edge_batch(C, keep, min_tok, max_keep):
    """sp_select_legacy on given chunk scores (many ties) for a batch of 20
    prompts from 1 to 5000 tokens: exactly the oracle's rule and cap."""
    lengths = [1, 2, 3, 4, 5, 6, 7, 9, 31, 33, 64, 100, 250, 1000, 3000, 5000, 17, 129, 4, 777]
    rng = np.random.default_rng(C * 1000 + max_keep)
    batch = sp.Batch(np.concatenate([[0], np.cumsum(lengths)]))
    means = [np.round(rng.random(-(-n // C)) * 4).astype(np.float32) / 4 for n in lengths]
    cs = torch.from_numpy(np.concatenate(means)).to(DEV)
    ids = torch.from_numpy(rng.integers(0, 1 << 17, batch.total).astype(np.int32)).to(DEV)
    kid, kpos, koff = sp.select_legacy(batch, C, keep, min_tok, max_keep, cs, ids)
    torch.cuda.synchronize()
    kid, kpos, koff = kid.cpu().numpy(), kpos.cpu().numpy(), koff.cpu().numpy()
    ids = ids.cpu().numpy()
    assert koff[0] == 0
    for b, n in enumerate(lengths):
        want = oracle.thin(oracle.select_legacy_from_means(means[b], n, C, keep, min_tok), max_keep)
        np.testing.assert_array_equal(kpos[koff[b]:koff[b + 1]], want, err_msg=f"prompt {b} n={n}")
        np.testing.assert_array_equal(kid[koff[b]:koff[b + 1]], ids[batch.offsets[b] + want])


# ----------------------------------------------------------------------------
# Gather on random keep flags: batches small enough for the one-launch kernel
# (<= 16384 chunks) and one past it (scan + write), every chunk size class.
# ----------------------------------------------------------------------------

GATHER_CASES = [
    # (lengths, C, p_keep, chunk 0 of every prompt dropped)
    ((1,), 32, 0.5, False),
    ((5000,), 1, 0.5, True),
    ((3, 1030, 2047, 64), 3, 0.4, True),
    ((131072,), 32, 0.8, True),
    ((70000, 1500, 33), 1000, 0.5, True),
    ((100, 4096, 999, 2049) * 8, 32, 0.3, False),
    ((33, 64, 97, 1, 500) * 25 + (40, 41, 2), 32, 0.5, True),   # 128 prompts
    ((300000, 250000), 32, 0.6, True),          # 17188 chunks: the two-kernel form
    ((4160,) * 127 + (77,), 32, 0.5, True),    # 128 prompts, 16513 chunks: two kernels
]


@pytest.mark.gpu
@pytest.mark.parametrize("lengths,C,p_keep,drop0", GATHER_CASES)
def test_gather_random_keep(lengths, C, p_keep, drop0):
    """Kept ids, positions and offsets against the oracle's gather, prompt by prompt."""
    rng = np.random.default_rng(len(lengths) * 1000 + C)
    lengths = list(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ncs = [(n + C - 1) // C for n in lengths]
    keep = []
    for nc in ncs:
        k = (rng.random(nc) < p_keep).astype(np.uint8)
        k[-1] = 1
        if drop0 and nc > 1:
            k[0] = 0
        keep.append(k)
    keep_all = np.concatenate(keep)
    ids = rng.integers(0, 1 << 30, size=int(off[-1]), dtype=np.int32)
    kid, kpos, koff = sp.sp_gather_kept(torch.from_numpy(keep_all).to(DEV),
                                        torch.from_numpy(ids).to(DEV), torch.from_numpy(off), C)
    torch.cuda.synchronize()
    kid, kpos, koff = kid.cpu().numpy(), kpos.cpu().numpy(), koff.cpu().numpy()
    assert koff[0] == 0
    for b, n in enumerate(lengths):
        want_ids, want_pos = oracle.gather(keep[b], ids[off[b]:off[b + 1]], C)
        assert koff[b + 1] - koff[b] == want_ids.size, (b, koff[b + 1] - koff[b], want_ids.size)
        assert np.array_equal(kid[koff[b]:koff[b + 1]], want_ids), b
        assert np.array_equal(kpos[koff[b]:koff[b + 1]], want_pos), b


# ----------------------------------------------------------------------------
# Pooling on random importance: block shapes (one token per thread up to
# C = 256, one chunk per block beyond), the compile-time 13-token window and
# the run-time one, prompt edges, with and without normalisation.
# ----------------------------------------------------------------------------

POOL_CASES = [
    # (lengths, W, C, normalize)
    ((5000, 7, 300), 13, 32, True),
    ((5000, 7, 300), 13, 32, False),
    ((4099,), 5, 7, True),
    ((3000, 257), 33, 256, True),
    ((3000, 600), 13, 257, True),
    ((2500,), 129, 1000, True),
    ((12, 13, 14), 13, 1, True),
    ((70000,), 1, 300, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("lengths,W,C,normalize", POOL_CASES)
def test_pool_chunk_random(lengths, W, C, normalize):
    """Token and chunk scores against the oracle's pooling, prompt by prompt."""
    rng = np.random.default_rng(W * 1000 + C)
    lengths = list(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    imp = (rng.random(int(off[-1])) ** 4).astype(np.float32)
    ts, cs = sp.sp_pool_chunk(torch.from_numpy(imp).to(DEV), torch.from_numpy(off), W=W, C=C,
                              normalize=normalize)
    torch.cuda.synchronize()
    ts, cs = ts.cpu().numpy(), cs.cpu().numpy()
    c0 = 0
    for b, n in enumerate(lengths):
        nc = (n + C - 1) // C
        want_ts, want_cs = oracle.pool_chunk(imp[off[b]:off[b + 1]].astype(np.float64), W=W, C=C,
                                             normalize=normalize)
        assert_scores_close(ts[off[b]:off[b + 1]], want_ts, f"token scores {b}")
        assert_scores_close(cs[c0:c0 + nc], want_cs, f"chunk scores {b}")
        c0 += nc
