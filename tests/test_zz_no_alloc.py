"""sp_score_attention_noalloc against sp_score_attention, through the C ABI.

The no-alloc entry point runs the same kernels with the library's own scratch
as workspace, so on the same inputs its importance must equal the allocating
call's bit for bit. Calls follow one another on the shared scratch with
smaller inputs after larger ones, and switch between the single pass and the
two-pass kernels, so a later call runs on what an earlier one left there.
"""
import ctypes

import pytest
import torch

import workloads
from draft_attention_token_amd import specprefill as sp

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _case(name, algo):
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    q, k = inp.q.to(DEV), inp.k.to(DEV)
    batch = sp.Batch(inp.offsets)
    desc = sp.attn_desc(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_lookahead, w.dtype,
                        algo=algo, k_dtype=inp.k.dtype, k_scales=inp.k_scales,
                        prefill_row=w.prefill_row)
    return w, q, k, batch, desc


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(name, algo, expect_kernel):
    w, q, k, batch, desc = _case(name, algo)
    print(f"no-alloc case {name} algo={algo}", flush=True)
    assert sp.score_plan(desc, batch).kernel == expect_kernel
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    ws = sp._ws(sp.score_workspace_bytes(desc, batch), DEV)
    ref = torch.full((batch.total,), float("nan"), dtype=torch.float32, device=DEV)
    rc = sp.lib().sp_score_attention(ctypes.byref(desc), batch.ref(), _ptr(q), _ptr(k), _ptr(ref),
                                     _ptr(ws), ws.numel(), st)
    assert rc == sp.SP_OK, sp.status_string(rc)
    out = torch.full((batch.total,), float("nan"), dtype=torch.float32, device=DEV)
    sp.sp_score_attention_noalloc(q, k, batch, desc, out)
    torch.cuda.synchronize()
    assert sp.score_status(ws) == 0
    assert torch.isfinite(ref).all() and torch.isfinite(out).all()
    assert torch.equal(out, ref), f"{name}: no-alloc importance differs from the allocating call"


def test_noalloc_matches_allocating_call_twice_then_smaller():
    # single pass on 32768 tokens, then on 3212 (smaller), then the two-pass
    # kernels on the same 3212 tokens (AUTO takes them for short batches)
    _both("n32k_bf16", "auto", "stream")
    _both("n3212_bf16", "stream", "stream")
    _both("n3212_bf16", "auto", "two_pass")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 8 layers x 16 KV heads = 128 (layer, KV head) pairs: the single pass
    # would need 256 B + 128 x 384 KiB > 48 MiB. Rejected before any launch.
    n = 4096
    batch = sp.Batch([0, n])
    desc = sp.attn_desc(8, 16, 16, 128, 1, torch.bfloat16, algo="stream")
    q = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(n, dtype=torch.float32, device=DEV)
    rc = sp.lib().sp_score_attention_noalloc(ctypes.byref(desc), batch.ref(),
                                             ctypes.c_void_p(q.data_ptr()),
                                             ctypes.c_void_p(q.data_ptr()),
                                             ctypes.c_void_p(out.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert rc == sp.SP_ERR_WORKSPACE_TOO_SMALL, sp.status_string(rc)
