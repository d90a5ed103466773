"""GPU parity of sp_pool_select_gather, the one-call form of the stages after
scoring (pooling, normalisation, boosts, chunk means, selection, compaction).

Its results must equal those of sp_pool_chunk, sp_select_chunks and
sp_gather_kept called one after the other, bit for bit (same arithmetic in
the same order), in each of its forms: the die-local launch (every chip die
runs the batch and finds the selection cutoff itself), the launch over the
whole chip, and the separate kernels; and, prompt by prompt, those of the
oracle's pooling, selection and gather within the parity tolerances.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from draft_attention_token_amd import specprefill as sp

from parity import assert_scores_close, check_prompt

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RAGGED16 = (65536, 2048, 40000, 8192, 30000, 4096, 50000, 12000, 20000, 6000, 60000, 3000, 25000,
            10000, 45000, 16384)

CASES = [
    # (lengths, W, C, normalize, importance kind)
    ((1,), 13, 32, True, "rand"),
    ((31, 32, 33, 97), 13, 32, True, "rand"),
    ((3212, 100, 5000), 13, 32, True, "spiky"),
    ((131072,), 13, 32, True, "rand"),                 # one prompt over every CU
    ((131072,), 13, 32, True, "ties"),
    ((163840,), 13, 32, True, "spiky"),
    (RAGGED16, 13, 32, True, "spiky"),
    ((4099, 17), 5, 7, True, "ties"),
    ((3000, 257), 33, 256, True, "rand"),
    ((2500,), 129, 1000, True, "rand"),
    ((5000, 7, 300), 13, 32, False, "rand"),
    ((20000,), 13, 32, True, "flat"),                  # no signal: every score 1, then boosts
    ((33, 64, 97, 1, 500) * 25 + (40, 41, 2), 13, 32, True, "rand"),   # 128 prompts
    ((60000,) * 4, 13, 8, True, "rand"),               # die-local, 7680-token ranges
    ((70000,) * 4, 13, 8, True, "rand"),               # fits neither one-launch form
    ((140000,), 13, 16, True, "spiky"),                # 8750 chunks: 16 scores per thread
    ((3000, 5000), 5, 1, True, "rand"),                # one-token chunks
    ((257, 1000, 33, 8000) * 8, 13, 32, True, "spiky"),  # 32 prompts: a die's every CU
]
MODES = [("top_p", 0.3), ("mass", 0.85), ("mass", 0.999)]


def _importance(kind, n, rng):
    if kind == "rand":
        return rng.random(n).astype(np.float32)
    if kind == "spiky":
        return (rng.random(n) ** 8).astype(np.float32)
    if kind == "ties":
        return (rng.integers(0, 4, n) / 4.0).astype(np.float32)
    return np.full(n, 0.25, dtype=np.float32)


def _inputs(lengths, kind, seed):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    imp = _importance(kind, int(off[-1]), rng)
    ids = rng.integers(0, 1 << 30, size=int(off[-1]), dtype=np.int32)
    return off, imp, ids


def _separate(imp_d, ids_d, batch, W, C, normalize, mode, param):
    ts, cs = sp.sp_pool_chunk(imp_d, batch, W=W, C=C, normalize=normalize)
    keep, cnt = sp.sp_select_chunks(cs, batch, C, mode, param)
    kid, kpos, koff = sp.sp_gather_kept(keep, ids_d, batch, C)
    return ts, cs, keep, cnt, kid, kpos, koff


def _assert_same(fused, sep, what):
    names = ["token_scores", "chunk_scores", "keep", "n_kept"]
    for name, a, b in zip(names, fused[:4], sep[:4]):
        assert torch.equal(a.cpu(), b.cpu()), f"{what}: {name} differ"
    koff_f, koff_s = fused[6].cpu(), sep[6].cpu()
    assert torch.equal(koff_f, koff_s), f"{what}: kept offsets differ"
    n = int(koff_s[-1])
    assert torch.equal(fused[4][:n].cpu(), sep[4][:n].cpu()), f"{what}: kept ids differ"
    assert torch.equal(fused[5][:n].cpu(), sep[5][:n].cpu()), f"{what}: kept positions differ"


@pytest.mark.parametrize("lengths, W, C, normalize, kind", CASES,
                         ids=[f"{len(c[0])}p_{sum(c[0])}t_W{c[1]}_C{c[2]}_{'n' if c[3] else 'raw'}_{c[4]}"
                              for c in CASES])
def test_one_call_equals_the_three_calls(lengths, W, C, normalize, kind):
    off, imp, ids = _inputs(lengths, kind, seed=sum(lengths) % 9973 + C)
    batch = sp.Batch(off)
    pd = sp.pool_desc(W, C, normalize)
    form, tb = sp.post_form(pd, batch)
    assert sp.post_plan(pd, batch) == tb
    print(f"[gpu] post {len(lengths)} prompts {sum(lengths)} tokens W={W} C={C} {kind}: "
          f"form {form}, block tokens {tb}", flush=True)
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    ws = sp._ws(sp.post_workspace_bytes(pd, batch), DEV)
    for mode, param in MODES:
        fused = sp.sp_pool_select_gather(imp_d, ids_d, batch, mode, param, W=W, C=C,
                                         normalize=normalize, ws=ws)
        sep = _separate(imp_d, ids_d, batch, W, C, normalize, mode, param)
        torch.cuda.synchronize()
        assert sp.score_status(ws) == 0, "a wait of the one-launch form timed out"
        _assert_same(fused, sep, f"{mode} {param}")


EDGE = [
    # (lengths, W, C, normalize, kind)
    ((512,), 13, 32, True, "rand"),                    # exactly one 512-token block
    ((1, 131071), 13, 32, True, "spiky"),              # a one-token prompt ahead of a long one
    ((131071, 1), 13, 32, True, "spiky"),              # and after it
    ((5000, 3000), 129, 1024, True, "rand"),           # widest window, largest chunk
    ((2048, 2047, 2049), 1, 32, True, "ties"),         # no pooling; block edges
    ((40000,), 13, 16, False, "spiky"),                # no normalisation, small chunks
]


@pytest.mark.parametrize("lengths, W, C, normalize, kind", EDGE,
                         ids=["one_block", "tiny_first", "tiny_last", "W129_C1024", "W1_edges",
                              "raw_C16"])
def test_one_call_edges(lengths, W, C, normalize, kind):
    off, imp, ids = _inputs(lengths, kind, seed=sum(lengths) % 7919 + W)
    batch = sp.Batch(off)
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    print(f"[gpu] post edge {lengths} W={W} C={C}: form, block tokens "
          f"{sp.post_form(sp.pool_desc(W, C, normalize), batch)}", flush=True)
    for mode, param in MODES:
        fused = sp.sp_pool_select_gather(imp_d, ids_d, batch, mode, param, W=W, C=C,
                                         normalize=normalize)
        sep = _separate(imp_d, ids_d, batch, W, C, normalize, mode, param)
        torch.cuda.synchronize()
        _assert_same(fused, sep, f"{mode} {param}")


def test_one_call_without_token_scores():
    """token_scores may be NULL: everything else is unchanged."""
    off, imp, ids = _inputs((3212, 100, 5000), "spiky", seed=3)
    batch = sp.Batch(off)
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    a = sp.sp_pool_select_gather(imp_d, ids_d, batch, "mass", 0.85)
    b = sp.sp_pool_select_gather(imp_d, ids_d, batch, "mass", 0.85, token_scores=False)
    torch.cuda.synchronize()
    assert b[0] is None
    for x, y in zip(a[1:4] + a[6:], b[1:4] + b[6:]):
        assert torch.equal(x, y)
    n = int(a[6][-1])
    assert torch.equal(a[4][:n], b[4][:n]) and torch.equal(a[5][:n], b[5][:n])


def test_forms_of_the_benchmark_batches():
    """One 128K prompt: the die-local form, one range per CU of a die (4096
    tokens at 32 CUs per die). The 16-prompt ragged batch of 397256 tokens
    needs more ranges than a die has CUs at 8192 tokens each: the grid form.
    More than 32 prompts: the grid form. Four 70000-token prompts of 8-token
    chunks are more than a die's ranges hold and need more grid blocks than
    the device has CUs: the separate kernels."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    pd = sp.pool_desc()
    form, tb = sp.post_form(pd, sp.Batch([0, 131072]))
    assert form == "die" and tb % 256 == 0 and (131072 + tb - 1) // tb <= cus // 8, (form, tb)
    off = np.concatenate([[0], np.cumsum(RAGGED16)])
    assert sp.post_form(pd, sp.Batch(off))[0] == "grid"
    assert sp.post_form(pd, sp.Batch(np.arange(0, 33 * 100 + 1, 100)))[0] == "grid"
    assert sp.post_form(pd, sp.Batch(np.arange(0, 32 * 100 + 1, 100)))[0] == "die"
    assert sp.post_form(sp.pool_desc(C=8), sp.Batch([0, 70000, 140000, 210000, 280000])) == \
        ("separate", 0)
    assert sp.post_form(sp.pool_desc(C=8), sp.Batch([0, 60000, 120000, 180000, 240000]))[0] == "die"


@pytest.mark.parametrize("lengths, W, C, normalize, kind", [CASES[2], CASES[7], CASES[12]],
                         ids=["3prompts", "C7_W5_ties", "128prompts"])
def test_one_call_against_the_oracle(lengths, W, C, normalize, kind):
    off, imp, ids = _inputs(lengths, kind, seed=77 + C)
    batch = sp.Batch(off)
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    for mode, param in MODES:
        ts, cs, keep, cnt, kid, kpos, koff = sp.sp_pool_select_gather(
            imp_d, ids_d, batch, mode, param, W=W, C=C, normalize=normalize)
        torch.cuda.synchronize()
        ts, cs, keep, cnt = ts.cpu().numpy(), cs.cpu().numpy(), keep.cpu().numpy(), cnt.cpu().numpy()
        kid, kpos, koff = kid.cpu().numpy(), kpos.cpu().numpy(), koff.cpu().numpy()
        ora = dict(token_scores=[], chunk_scores=[], keep=[], kept_ids=[], kept_pos=[])
        for b in range(len(lengths)):
            t, c = oracle.pool_chunk(imp[off[b]:off[b + 1]].astype(np.float64), W=W, C=C,
                                     normalize=normalize)
            k = oracle.select(c, mode, param)
            i, p = oracle.gather(k, ids[off[b]:off[b + 1]], C)
            for key, v in zip(ora, (t, c, k, i, p)):
                ora[key].append(v)
        c0 = 0
        assert koff[0] == 0
        for b, n in enumerate(lengths):
            nc = (n + C - 1) // C
            assert_scores_close(ts[off[b]:off[b + 1]], ora["token_scores"][b], f"token scores {b}")
            gpu = dict(chunk_scores=cs[c0:c0 + nc], keep=keep[c0:c0 + nc],
                       kept_ids=kid[koff[b]:koff[b + 1]], kept_pos=kpos[koff[b]:koff[b + 1]])
            check_prompt(gpu, ora, b, mode, param, C, ids[off[b]:off[b + 1]])
            assert cnt[b] == int(gpu["keep"].sum())
            c0 += nc


@pytest.mark.parametrize("lengths, form", [((131072,), "die"), ((70000, 3000, 60000), "die"),
                                           (RAGGED16, "grid")], ids=["die", "die_3p", "grid"])
def test_timed_out_call_reports_and_the_workspace_stays_usable(monkeypatch, lengths, form):
    """A zero wait budget (SP_SCORE_WAIT_US=0, read at launch) lets a block
    give up on any value not already posted: the grid still drains, and the
    call either completed anyway or reports the time-out (and then wrote no
    kept tokens). The next call on the same workspace, with the normal
    budget, matches the separate kernels bit for bit."""
    off, imp, ids = _inputs(lengths, "rand", seed=5)
    batch = sp.Batch(off)
    pd = sp.pool_desc()
    assert sp.post_form(pd, batch)[0] == form
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    ws = sp._ws(sp.post_workspace_bytes(pd, batch), DEV)
    sep = _separate(imp_d, ids_d, batch, 13, 32, True, "mass", 0.85)
    monkeypatch.setenv("SP_SCORE_WAIT_US", "0")
    print("[gpu] one-call post with a zero wait budget", flush=True)
    first = sp.sp_pool_select_gather(imp_d, ids_d, batch, "mass", 0.85, ws=ws)
    torch.cuda.synchronize()
    if sp.score_status(ws) == 0:
        _assert_same(first, sep, "zero budget, no time-out")
    monkeypatch.delenv("SP_SCORE_WAIT_US")
    again = sp.sp_pool_select_gather(imp_d, ids_d, batch, "mass", 0.85, ws=ws)
    torch.cuda.synchronize()
    assert sp.score_status(ws) == 0
    _assert_same(again, sep, "after a zero-budget call")


def test_separate_form_clears_the_status_of_an_earlier_call():
    """The status header of a call that runs the separate kernels says
    'completed' even on a workspace whose previous call timed out."""
    pd = sp.pool_desc(C=8)
    off, imp, ids = _inputs((70000,) * 4, "rand", seed=8)
    batch = sp.Batch(off)
    assert sp.post_plan(pd, batch) == 0
    ws = sp._ws(sp.post_workspace_bytes(pd, batch), DEV)
    ws[:8].copy_(torch.tensor([7, 0, 0, 0, 7, 0, 0, 0], dtype=torch.uint8))   # [0] == [1]: failed
    assert sp.score_status(ws) == 1
    imp_d, ids_d = torch.from_numpy(imp).to(DEV), torch.from_numpy(ids).to(DEV)
    sp.sp_pool_select_gather(imp_d, ids_d, batch, "top_p", 0.3, C=8, ws=ws)
    torch.cuda.synchronize()
    assert sp.score_status(ws) == 0


def test_pipeline_forms_agree():
    """Pipeline.run with the one call and with the three calls."""
    import workloads
    w = workloads.small_workload("n3212_bf16", lengths=(3212, 100, 5000), seed=21)
    inp = workloads.make_inputs(w)
    q, k, ids = inp.q.to(DEV), inp.k.to(DEV), inp.token_ids.to(DEV)
    pipes = []
    for fused in (True, False):
        p = sp.Pipeline(inp.offsets, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim,
                        w.n_lookahead, w.dtype, DEV, mode="mass", param=0.85, fused=fused)
        p.run(q, k, ids, check=True)
        pipes.append(p)
    torch.cuda.synchronize()
    a, b = pipes
    for name in ("importance", "token_scores", "chunk_scores", "keep", "n_kept", "kept_offsets"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    n = int(b.kept_offsets[-1])
    assert torch.equal(a.kept_ids[:n], b.kept_ids[:n])
    assert torch.equal(a.kept_pos[:n], b.kept_pos[:n])
