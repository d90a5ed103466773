"""Pins of the CPU oracle against facts other than itself.

Each test checks the oracle against something the pages or mathematics fix:
closed forms, invariants, library routines on tiny shapes, exhaustive search,
and the kept-token counts printed on the pull-request page. None of these
needs a GPU.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, lengths, n_layers, Hq, Hkv, d, L, scale_q=1.0):
    B = len(lengths)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    q = (rng.standard_normal((B, n_layers, L, Hq, d)) * scale_q).astype(np.float32)
    k = rng.standard_normal((n_layers, int(off[-1]) + B * L, Hkv, d)).astype(np.float32)
    return off, q, k


def _importance_bruteforce(off, q, k, n_layers, Hq, Hkv, d, L, scale):
    """Independent route: dense logits via numpy, masked softmax via scipy,
    reductions via numpy max/mean over named axes."""
    B = len(off) - 1
    G = Hq // Hkv
    out = []
    for b in range(B):
        n = int(off[b + 1] - off[b])
        k0 = int(off[b]) + b * L
        kb = k[:, k0:k0 + n + L].astype(np.float64)            # [l][key][g][d]
        kq = np.repeat(kb, G, axis=2)                           # [l][key][h][d]
        qb = q[b].astype(np.float64)                            # [l][j][h][d]
        s = np.einsum("ljhd,lkhd->ljhk", qb, kq) * scale        # [l][j][h][key]
        key_pos = np.arange(n + L)
        mask = key_pos[None, :] <= (n + np.arange(L))[:, None]  # [j][key]
        s = np.where(mask[None, :, None, :], s, -np.inf)
        p = scipy.special.softmax(s, axis=-1)[..., :n]          # prompt columns
        stepmax = p.max(axis=2).max(axis=0)                     # heads, then layers -> [j][k]
        out.append(stepmax.mean(axis=0))
    return np.concatenate(out)


# ----------------------------------------------------------------------------
# Softmax rows and importance
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(0)
    off, q, k = _rand_problem(rng, [7, 12], 2, 4, 2, 8, 3, scale_q=2.0)
    scale = 1 / math.sqrt(8)
    for (b, l, j, h) in itertools.product(range(2), range(2), range(3), range(4)):
        p = oracle.softmax_row(off, q, k, 2, 4, 2, 8, 3, scale, b, l, j, h)
        n = off[b + 1] - off[b]
        assert p.size == n + j + 1
        assert abs(p.sum() - 1.0) < 1e-12
        k0 = int(off[b]) + b * 3
        s = k[l, k0:k0 + n + j + 1, h // 2, :].astype(np.float64) @ q[b, l, j, h].astype(np.float64)
        np.testing.assert_allclose(p, scipy.special.softmax(s * scale), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("shape", [
    dict(lengths=[5], n_layers=1, Hq=1, Hkv=1, d=4, L=1),
    dict(lengths=[9, 4, 13], n_layers=3, Hq=4, Hkv=2, d=8, L=3),
    dict(lengths=[17], n_layers=2, Hq=8, Hkv=2, d=16, L=8),
    dict(lengths=[6, 11], n_layers=2, Hq=6, Hkv=3, d=4, L=2),
])
def test_importance_matches_bruteforce(shape):
    rng = np.random.default_rng(1)
    off, q, k = _rand_problem(rng, shape["lengths"], shape["n_layers"], shape["Hq"],
                              shape["Hkv"], shape["d"], shape["L"], scale_q=3.0)
    scale = 1 / math.sqrt(shape["d"])
    args = (shape["n_layers"], shape["Hq"], shape["Hkv"], shape["d"], shape["L"], scale)
    got = oracle.importance(off, q, k, *args)
    ref = _importance_bruteforce(off, q, k, *args)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_importance_all_zero_q_is_uniform_closed_form():
    """Zero queries give uniform rows: p = 1/(N+j+1), so
    imp = (1/L) * sum_j 1/(N+j+1) at every prompt position."""
    rng = np.random.default_rng(2)
    lengths, L = [50, 33], 8
    off, q, k = _rand_problem(rng, lengths, 3, 4, 1, 16, L)
    q[:] = 0
    imp = oracle.importance(off, q, k, 3, 4, 1, 16, L, 0.25)
    for b, n in enumerate(lengths):
        want = sum(1.0 / (n + j + 1) for j in range(L)) / L
        np.testing.assert_allclose(imp[off[b]:off[b + 1]], want, rtol=1e-14)


def test_importance_single_hot_prompt_key_closed_form():
    """All keys zero except key k0 of group 0, whose logit is `a` for every
    query of group 0. Group-0 rows: p(k0) = e^a/(e^a+N+j), others
    1/(e^a+N+j); group-1 rows are uniform 1/(N+j+1)."""
    n, L, d, a, k0 = 40, 4, 8, 2.5, 17
    off = np.array([0, n], dtype=np.int64)
    q = np.zeros((1, 2, L, 4, d), dtype=np.float32)   # 2 layers, Hq=4, Hkv=2
    k = np.zeros((2, n + L, 2, d), dtype=np.float32)
    k[:, k0, 0, 0] = 1.0
    scale = 0.5
    q[:, :, :, 0:2, 0] = a / scale                     # group-0 heads
    imp = oracle.importance(off, q, k, 2, 4, 2, d, L, scale)
    ea = math.exp(a)
    want_hot = sum(ea / (ea + n + j) for j in range(L)) / L
    want_cold = sum(1.0 / (n + j + 1) for j in range(L)) / L
    assert abs(imp[k0] - want_hot) < 1e-14
    others = np.delete(imp, k0)
    np.testing.assert_allclose(others, want_cold, rtol=1e-14)


def test_importance_causal_lookahead_key_closed_form():
    """A hot key at lookahead position N+2 is seen only by queries j >= 2.
    With one KV group, prompt keys get 1/(N+j+1) for j < 2 and
    1/(e^a+N+j) for j >= 2."""
    n, L, d, a = 30, 5, 4, 3.0
    off = np.array([0, n], dtype=np.int64)
    q = np.zeros((1, 1, L, 2, d), dtype=np.float32)   # 1 layer, Hq=2, Hkv=1
    k = np.zeros((1, n + L, 1, d), dtype=np.float32)
    k[0, n + 2, 0, 0] = 1.0
    q[0, 0, :, :, 0] = a                                # scale 1
    imp = oracle.importance(off, q, k, 1, 2, 1, d, L, 1.0)
    ea = math.exp(a)
    want = (sum(1.0 / (n + j + 1) for j in range(2)) + sum(1.0 / (ea + n + j) for j in range(2, L))) / L
    np.testing.assert_allclose(imp, want, rtol=1e-14)


def test_importance_invariant_to_layer_and_head_permutations():
    rng = np.random.default_rng(3)
    n_layers, Hq, Hkv, d, L = 3, 6, 3, 8, 4
    off, q, k = _rand_problem(rng, [21, 10], n_layers, Hq, Hkv, d, L, scale_q=2.0)
    args = (n_layers, Hq, Hkv, d, L, 0.3)
    base = oracle.importance(off, q, k, *args)
    # permute layers
    perm = [2, 0, 1]
    np.testing.assert_allclose(oracle.importance(off, q[:, perm], k[perm], *args), base, rtol=1e-14)
    # permute q-heads inside each group (G = 2)
    hp = [1, 0, 3, 2, 5, 4]
    np.testing.assert_allclose(oracle.importance(off, q[:, :, :, hp], k, *args), base, rtol=1e-14)
    # permute KV groups together with their q-heads
    gp = [2, 0, 1]
    hp2 = [h for g in gp for h in (2 * g, 2 * g + 1)]
    np.testing.assert_allclose(oracle.importance(off, q[:, :, :, hp2], k[:, :, gp], *args), base,
                               rtol=1e-14)
    # duplicating a layer leaves the max over layers unchanged
    q2 = np.concatenate([q, q[:, :1]], axis=1)
    k2 = np.concatenate([k, k[:1]], axis=0)
    np.testing.assert_allclose(oracle.importance(off, q2, k2, n_layers + 1, Hq, Hkv, d, L, 0.3),
                               base, rtol=1e-14)


def test_importance_prompts_are_independent():
    """A prompt's scores do not depend on the other prompts of the batch."""
    rng = np.random.default_rng(4)
    off, q, k = _rand_problem(rng, [12, 20], 2, 4, 2, 8, 3)
    both = oracle.importance(off, q, k, 2, 4, 2, 8, 3, 0.4)
    k1 = np.ascontiguousarray(k[:, 15:15 + 23])
    one = oracle.importance(np.array([0, 20]), q[1:], k1, 2, 4, 2, 8, 3, 0.4)
    np.testing.assert_allclose(both[12:], one, rtol=1e-15)


def test_importance_does_not_depend_on_the_thread_count():
    """The max over layers and heads is merged from parallel tasks; maxima
    are exact in any order, so every thread count gives the same bits."""
    rng = np.random.default_rng(41)
    off, q, k = _rand_problem(rng, [40, 7, 65], 3, 4, 2, 8, 4)
    one = oracle.importance(off, q, k, 3, 4, 2, 8, 4, 0.35, nthreads=1)
    for n in (2, 3, 8):
        assert np.array_equal(oracle.importance(off, q, k, 3, 4, 2, 8, 4, 0.35, nthreads=n), one)


# ----------------------------------------------------------------------------
# Pool-before-max: each probability row pooled before the head/layer max
# ----------------------------------------------------------------------------

def _box_counts(n, W):
    """Centred window sums via numpy.convolve ("full", then the centred
    slice, which also holds for n < W), divided by the in-range count."""
    ones, r = np.ones(W), (W - 1) // 2
    cnt = np.convolve(np.ones(n), ones)[r:r + n]
    return lambda x: np.convolve(x, ones)[r:r + n] / cnt


def test_row_pool_width_one_is_the_plain_importance():
    rng = np.random.default_rng(31)
    off, q, k = _rand_problem(rng, [30, 11], 2, 4, 2, 8, 3, scale_q=2.0)
    a = oracle.importance(off, q, k, 2, 4, 2, 8, 3, 0.4)
    b = oracle.importance(off, q, k, 2, 4, 2, 8, 3, 0.4, row_pool=1)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("W", [3, 13])
def test_row_pool_matches_bruteforce(W):
    """Dense softmax, numpy.convolve on each row's prompt columns, then the
    max over heads and layers and the mean over steps."""
    rng = np.random.default_rng(32)
    n_layers, Hq, Hkv, d, L = 2, 8, 2, 8, 3
    lengths = [40, 5, 19]
    off, q, k = _rand_problem(rng, lengths, n_layers, Hq, Hkv, d, L, scale_q=3.0)
    scale = 1 / math.sqrt(d)
    got = oracle.importance(off, q, k, n_layers, Hq, Hkv, d, L, scale, row_pool=W)
    G = Hq // Hkv
    for b, n in enumerate(lengths):
        k0 = int(off[b]) + b * L
        kb = np.repeat(k[:, k0:k0 + n + L].astype(np.float64), G, axis=2)
        s = np.einsum("ljhd,lkhd->ljhk", q[b].astype(np.float64), kb) * scale
        vis = np.arange(n + L)[None, :] <= (n + np.arange(L))[:, None]
        s = np.where(vis[None, :, None, :], s, -np.inf)
        p = scipy.special.softmax(s, axis=-1)[..., :n]
        pool = _box_counts(n, W)
        pooled = np.apply_along_axis(pool, -1, p)
        want = pooled.max(axis=2).max(axis=0).mean(axis=0)
        np.testing.assert_allclose(got[off[b]:off[b + 1]], want, rtol=1e-12, atol=1e-15)


def test_row_pool_all_zero_q_keeps_the_uniform_closed_form():
    """Uniform rows stay uniform under a count-normalised pool."""
    rng = np.random.default_rng(33)
    lengths, L = [50, 7], 4
    off, q, k = _rand_problem(rng, lengths, 2, 4, 1, 8, L)
    q[:] = 0
    imp = oracle.importance(off, q, k, 2, 4, 1, 8, L, 0.25, row_pool=13)
    for b, n in enumerate(lengths):
        want = sum(1.0 / (n + j + 1) for j in range(L)) / L
        np.testing.assert_allclose(imp[off[b]:off[b + 1]], want, rtol=1e-13)


def test_row_pool_single_hot_key_closed_form():
    """One hot key k0 (logit a) seen by the group-0 heads only. Group-0 rows:
    p(k0) = e^a / D_j, every other key 1 / D_j, with D_j = e^a + N + j. Pooled
    with W = 13, a key within 6 of k0 averages (e^a + 12) / (13 D_j) (interior
    keys); farther keys stay at 1 / D_j, below group 1's uniform 1/(N + j + 1),
    which the max then picks."""
    n, L, d, a, k0, W = 60, 3, 8, 3.0, 30, 13
    off = np.array([0, n], dtype=np.int64)
    q = np.zeros((1, 1, L, 4, d), dtype=np.float32)   # 1 layer, Hq=4, Hkv=2
    k = np.zeros((1, n + L, 2, d), dtype=np.float32)
    k[0, k0, 0, 0] = 1.0
    q[0, 0, :, 0:2, 0] = a
    imp = oracle.importance(off, q, k, 1, 4, 2, d, L, 1.0, row_pool=W)
    ea = math.exp(a)
    near = sum(max((ea + 12) / (13 * (ea + n + j)), 1.0 / (n + j + 1)) for j in range(L)) / L
    far = sum(1.0 / (n + j + 1) for j in range(L)) / L
    assert (ea + 12) / 13 > 1.0                       # the pooled hot window wins the max
    for kk in range(n):
        want = near if abs(kk - k0) <= 6 else far
        assert abs(imp[kk] - want) < 1e-14, kk


def test_row_pool_differs_from_pool_after():
    """The two orders are different functions (the max does not commute with
    the pool): on random rows they disagree."""
    rng = np.random.default_rng(34)
    off, q, k = _rand_problem(rng, [80], 2, 8, 2, 8, 4, scale_q=3.0)
    before = oracle.importance(off, q, k, 2, 8, 2, 8, 4, 0.35, row_pool=13)
    after, _ = oracle.pool_chunk(oracle.importance(off, q, k, 2, 8, 2, 8, 4, 0.35), 13, 32,
                                 False, 0, 1.0, 0, 1.0)
    assert np.abs(before - after).max() > 1e-4
    assert np.all(before <= after + 1e-15)   # max of means <= mean of maxes


# ----------------------------------------------------------------------------
# Prefill row: the prompt's own last row as one more step in front
# ----------------------------------------------------------------------------

def _prerow_problem(rng, lengths, n_layers, Hq, Hkv, d, L, scale_q=2.0):
    """Q with L + 1 steps, K with L lookahead keys per prompt."""
    B = len(lengths)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    q = (rng.standard_normal((B, n_layers, L + 1, Hq, d)) * scale_q).astype(np.float32)
    k = rng.standard_normal((n_layers, int(off[-1]) + B * L, Hkv, d)).astype(np.float32)
    return off, q, k


def test_prefill_row_all_zero_q_closed_form():
    """Zero queries: step j sees N + j keys (step 0 the N prompt keys), so
    imp = (1/(L+1)) * sum_{j=0..L} 1/(N + j)."""
    rng = np.random.default_rng(21)
    lengths, L = [40, 17], 5
    off, q, k = _prerow_problem(rng, lengths, 2, 4, 2, 8, L)
    q[:] = 0
    imp = oracle.importance(off, q, k, 2, 4, 2, 8, L, 0.3, prefill_row=True)
    for b, n in enumerate(lengths):
        want = sum(1.0 / (n + j) for j in range(L + 1)) / (L + 1)
        np.testing.assert_allclose(imp[off[b]:off[b + 1]], want, rtol=1e-14)


def test_prefill_row_is_a_shifted_lookahead_prompt():
    """The same Q and K read as a prompt one token shorter with one more
    lookahead key give the same rows: the first N - 1 scores agree, and only
    the last prompt token (a lookahead key there) is new."""
    rng = np.random.default_rng(22)
    n_layers, Hq, Hkv, d, L = 2, 8, 2, 8, 3
    lengths = [23, 9, 31]
    off, q, k = _prerow_problem(rng, lengths, n_layers, Hq, Hkv, d, L)
    pre = oracle.importance(off, q, k, n_layers, Hq, Hkv, d, L, 0.35, prefill_row=True)
    short = np.concatenate([[0], np.cumsum([n - 1 for n in lengths])]).astype(np.int64)
    plain = oracle.importance(short, q, k, n_layers, Hq, Hkv, d, L + 1, 0.35)
    for b, n in enumerate(lengths):
        np.testing.assert_allclose(pre[off[b]:off[b] + n - 1], plain[short[b]:short[b + 1]],
                                   rtol=1e-13, atol=1e-16)


def test_prefill_row_matches_bruteforce():
    """Dense route: step j of prompt b sits at position N - 1 + j."""
    rng = np.random.default_rng(23)
    n_layers, Hq, Hkv, d, L = 2, 4, 2, 8, 2
    lengths = [11, 6]
    off, q, k = _prerow_problem(rng, lengths, n_layers, Hq, Hkv, d, L)
    scale = 0.4
    got = oracle.importance(off, q, k, n_layers, Hq, Hkv, d, L, scale, prefill_row=True)
    G = Hq // Hkv
    for b, n in enumerate(lengths):
        k0 = int(off[b]) + b * L
        kb = np.repeat(k[:, k0:k0 + n + L].astype(np.float64), G, axis=2)   # [l][key][h][d]
        s = np.einsum("ljhd,lkhd->ljhk", q[b].astype(np.float64), kb) * scale
        vis = np.arange(n + L)[None, :] <= (n - 1 + np.arange(L + 1))[:, None]
        s = np.where(vis[None, :, None, :], s, -np.inf)
        p = scipy.special.softmax(s, axis=-1)[..., :n]
        want = p.max(axis=2).max(axis=0).mean(axis=0)
        np.testing.assert_allclose(got[off[b]:off[b + 1]], want, rtol=1e-12, atol=1e-15)


def test_prefill_row_alone():
    """With no lookahead keys the prefill row is the only step: its
    importance is the row's own softmax over the prompt, maxed over heads and
    layers."""
    rng = np.random.default_rng(24)
    off, q, k = _prerow_problem(rng, [15], 2, 4, 1, 8, 0)
    got = oracle.importance(off, q, k, 2, 4, 1, 8, 0, 0.5, prefill_row=True)
    rows = [oracle.softmax_row(off, q, k, 2, 4, 1, 8, 0, 0.5, 0, l, 0, h, prefill_row=True)
            for l in range(2) for h in range(4)]
    assert all(r.size == 15 for r in rows)
    np.testing.assert_allclose(got, np.max(rows, axis=0), rtol=1e-15)


# ----------------------------------------------------------------------------
# Quantised draft keys: fp8 e4m3 codes with a per-(layer, KV head) scale
# ----------------------------------------------------------------------------

def _e4m3fn_value(code):
    """OCP 8-bit e4m3 ("fn" variant): sign, 4 exponent bits with bias 7,
    3 mantissa bits, subnormals at exponent 0, no infinities, S.1111.111 NaN."""
    sgn = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return sgn * m * 2.0 ** -9
    return sgn * (1 + m / 8) * 2.0 ** (e - 7)


def test_fp8_codes_widen_per_the_format_definition():
    """The oracle widens K through torch's float8_e4m3fn; every one of the
    256 codes must give the value the format defines (448 the largest)."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = oracle._as_f32(codes).astype(np.float64)
    want = np.array([_e4m3fn_value(c) for c in range(256)])
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert want[0x7E] == 448.0 and want[0x01] == 2.0 ** -9 and want[0x38] == 1.0


def _rand_fp8_problem(rng, lengths, n_layers, Hq, Hkv, d, L):
    off, q, k = _rand_problem(rng, lengths, n_layers, Hq, Hkv, d, L, scale_q=2.0)
    codes, scales = workloads.quantize_fp8(torch.from_numpy(k))
    return off, q, codes, scales


def test_fp8_importance_matches_bruteforce_on_widened_keys():
    """Codes with scales equal the brute-force route on keys written out as
    scale * value(code) (values from the format definition, not torch)."""
    rng = np.random.default_rng(11)
    n_layers, Hq, Hkv, d, L = 2, 8, 2, 16, 4
    off, q, codes, scales = _rand_fp8_problem(rng, [19, 7, 30], n_layers, Hq, Hkv, d, L)
    table = np.array([_e4m3fn_value(c) for c in range(256)])
    vals = table[codes.view(torch.uint8).numpy().astype(np.int64)]
    assert not np.isnan(vals).any()
    keys = vals * scales.numpy().astype(np.float64)[:, None, :, None]
    scale = 1 / math.sqrt(d)
    got = oracle.importance(off, q, codes, n_layers, Hq, Hkv, d, L, scale, k_scales=scales)
    ref = _importance_bruteforce(off, q, keys, n_layers, Hq, Hkv, d, L, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_fp8_key_scale_is_a_logit_temperature():
    """Scaling problem (l, g)'s key scale by c scales that problem's logits by c:
    with one layer and one KV group, that is the plain scale times c."""
    rng = np.random.default_rng(12)
    off, q, codes, scales = _rand_fp8_problem(rng, [25, 9], 1, 4, 1, 8, 3)
    c = 2.0 ** 0.5
    ks = scales.double().numpy() * c                  # fp64: no rounding of the product
    a = oracle.importance(off, q, codes, 1, 4, 1, 8, 3, 0.3, k_scales=ks)
    b = oracle.importance(off, q, codes, 1, 4, 1, 8, 3, 0.3 * c * float(scales[0, 0]))
    np.testing.assert_allclose(a, b, rtol=1e-12)


def test_fp8_unit_scales_equal_plain_keys():
    """k_scales of one make the codes the keys."""
    rng = np.random.default_rng(13)
    off, q, codes, scales = _rand_fp8_problem(rng, [14], 2, 4, 2, 8, 2)
    ones = np.ones(scales.numel())
    a = oracle.importance(off, q, codes, 2, 4, 2, 8, 2, 0.25, k_scales=ones)
    b = oracle.importance(off, q, codes.to(torch.float32), 2, 4, 2, 8, 2, 0.25)
    np.testing.assert_array_equal(a, b)


def test_fp8_scale_index_is_layer_major():
    """Scale s[l][g] applies to layer l, KV group g only: raising one scale
    moves that problem's rows and leaves a problem it does not touch alone."""
    rng = np.random.default_rng(14)
    n_layers, Hq, Hkv, d, L = 2, 4, 2, 8, 2
    off, q, codes, scales = _rand_fp8_problem(rng, [12], n_layers, Hq, Hkv, d, L)
    base = scales.clone()
    hot = scales.clone()
    hot[1, 0] *= 3.0                                  # layer 1, group 0
    for (l, j, h) in itertools.product(range(n_layers), range(L), range(Hq)):
        p0 = oracle.softmax_row(off, q, codes, n_layers, Hq, Hkv, d, L, 0.3, 0, l, j, h,
                                k_scales=base)
        p1 = oracle.softmax_row(off, q, codes, n_layers, Hq, Hkv, d, L, 0.3, 0, l, j, h,
                                k_scales=hot)
        touched = l == 1 and h // (Hq // Hkv) == 0
        assert (np.abs(p0 - p1).max() > 1e-6) == touched, (l, j, h)


# ----------------------------------------------------------------------------
# Pooling, normalisation, boosts, chunk means
# ----------------------------------------------------------------------------

def test_pool_window_one_is_identity():
    x = np.random.default_rng(5).random(77)
    ts, cs = oracle.pool_chunk(x, W=1, C=32, normalize=False, first_mult=1.0, last_mult=1.0)
    np.testing.assert_array_equal(ts, x)
    np.testing.assert_allclose(cs, [x[0:32].mean(), x[32:64].mean(), x[64:77].mean()], rtol=1e-15)


def test_pool_constant_and_impulse():
    ts, _ = oracle.pool_chunk(np.full(40, 0.25), W=13, normalize=False, first_mult=1.0, last_mult=1.0)
    np.testing.assert_allclose(ts, 0.25, rtol=1e-15)
    n, k0 = 40, 3
    x = np.zeros(n)
    x[k0] = 1.0
    ts, _ = oracle.pool_chunk(x, W=13, normalize=False, first_mult=1.0, last_mult=1.0)
    for t in range(n):
        lo, hi = max(0, t - 6), min(n - 1, t + 6)
        want = 1.0 / (hi - lo + 1) if lo <= k0 <= hi else 0.0
        assert abs(ts[t] - want) < 1e-15


def test_pool_matches_numpy_convolve():
    x = np.random.default_rng(6).random(300)
    ts, _ = oracle.pool_chunk(x, W=13, normalize=False, first_mult=1.0, last_mult=1.0)
    sums = np.convolve(x, np.ones(13), mode="same")
    counts = np.convolve(np.ones_like(x), np.ones(13), mode="same")
    np.testing.assert_allclose(ts, sums / counts, rtol=1e-13)
    assert counts[0] == 7 and counts[6] == 13 and counts[-1] == 7


def test_normalise_then_boost_hand_values():
    """Constant scores carry no signal -> 1.0; then boosts: first 64 x1.5,
    last 128 x1.3. N=3212 puts the boost edge 12 tokens into chunk 96."""
    n = 3212
    _, cs = oracle.pool_chunk(np.full(n, 0.37), W=13, C=32, normalize=True)
    assert cs.size == 101
    np.testing.assert_allclose(cs[:2], 1.5, rtol=1e-15)
    np.testing.assert_allclose(cs[2:96], 1.0, rtol=1e-15)
    assert abs(cs[96] - (12 * 1.0 + 20 * 1.3) / 32) < 1e-15
    np.testing.assert_allclose(cs[97:], 1.3, rtol=1e-15)
    # min-max scaling of a ramp, W=1, no boosts
    x = np.arange(10, dtype=np.float64) * 2.0 + 5.0
    ts, _ = oracle.pool_chunk(x, W=1, C=4, normalize=True, first_mult=1.0, last_mult=1.0)
    np.testing.assert_allclose(ts, np.arange(10) / 9.0, rtol=1e-15)


def test_overlapping_boosts_multiply():
    ts, _ = oracle.pool_chunk(np.ones(100), W=1, C=32, normalize=False)
    np.testing.assert_allclose(ts[:64], 1.5 * 1.3)        # n < 192: all of 0..63 in both
    np.testing.assert_allclose(ts[64:], 1.3)


def test_pool_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.pool_chunk(np.ones(10), W=12)
    with pytest.raises(ValueError):
        oracle.pool_chunk(np.ones(10), C=0)


# ----------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------

def _order_key(cs, i):
    return (-cs[i], i)


def _best_set(cs, cands):
    """The candidate whose members, listed in selection order, are
    lexicographically first."""
    return min(cands, key=lambda s: sorted(_order_key(cs, i) for i in s))


@pytest.mark.parametrize("seed", range(12))
def test_top_p_matches_exhaustive_search(seed):
    rng = np.random.default_rng(100 + seed)
    nc = int(rng.integers(1, 11))
    cs = rng.integers(0, 4, nc).astype(np.float64)       # small value set -> ties
    for p in (0.05, 0.15, 0.3, 0.5, 0.77, 1.0):
        kc = oracle.top_p_count(nc, p)
        assert kc == max(1, min(nc, math.ceil(p * nc - 1e-9)))
        cands = [set(c) | {nc - 1} for c in itertools.combinations(range(nc - 1), kc - 1)]
        want = _best_set(cs, cands)
        keep = oracle.select(cs, "top_p", p)
        assert set(np.nonzero(keep)[0]) == want


@pytest.mark.parametrize("seed", range(12))
def test_mass_matches_exhaustive_search(seed):
    """Smallest set containing the final chunk whose mass reaches
    mass * total; among those, the first in selection order. Integer scores
    keep every sum exact."""
    rng = np.random.default_rng(200 + seed)
    nc = int(rng.integers(1, 11))
    cs = rng.integers(0, 5, nc).astype(np.float64)
    total = cs.sum()
    for m in (0.1, 0.5, 0.85, 0.9, 1.0):
        want = None
        for size in range(1, nc + 1):
            cands = [set(c) | {nc - 1} for c in itertools.combinations(range(nc - 1), size - 1)]
            ok = [s for s in cands if sum(cs[i] for i in s) >= m * total]
            if ok:
                want = _best_set(cs, ok)
                break
        keep = oracle.select(cs, "mass", m)
        assert set(np.nonzero(keep)[0]) == want


def _golden_counts():
    rows = []
    with open(os.path.join(GOLDEN, "pr_kept_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, p, kept = line.split()
                rows.append((int(n), float(p), int(kept)))
    return rows


def test_golden_kept_counts_from_pull_request():
    """Reproduce the 23 printed (N, p, kept) triples. The printed count is
    (kc - 1) full chunks + the final (partial) chunk, plus one BOS token when
    chunk 0 is not among the kept chunks; scores are built to put chunk 0
    in or out as the printed count implies, and the oracle's own selection
    and compaction must then give exactly the printed count."""
    rows = _golden_counts()
    assert len(rows) == 23
    C = 32
    for n, p, kept in rows:
        nc = (n + C - 1) // C
        kc = oracle.top_p_count(nc, p)
        tail = n - (nc - 1) * C
        base = (kc - 1) * C + tail
        extra = kept - base
        assert extra in (0, 1), (n, p, kept, kc)
        bos_separate = extra == 1
        assert not (bos_separate and kc == nc)
        # scores: descending with index except that chunk 0 is placed last
        # when BOS must come on its own, first otherwise.
        cs = np.linspace(1.0, 0.5, nc)
        cs[0] = 0.0 if bos_separate else 2.0
        keep = oracle.select(cs, "top_p", p)
        ids = np.arange(n, dtype=np.int32) + 1000
        ki, kp = oracle.gather(keep, ids, C)
        assert ki.size == kept, (n, p, kept)
        assert kp[0] == 0 and np.all(np.diff(kp) > 0)


def test_golden_counts_reject_other_rules():
    """The printed counts rule out neighbouring readings: rounding to nearest
    or down instead of up, and a final chunk kept on top of the budget."""
    rows = _golden_counts()
    C = 32

    def count(n, kc, chunk0_in):
        nc = (n + C - 1) // C
        tail = n - (nc - 1) * C
        return (kc - 1) * C + tail + (0 if chunk0_in or kc == nc else 1)

    def consistent(kc_fn, on_top=False):
        for n, p, kept in rows:
            nc = (n + C - 1) // C
            kc = kc_fn(nc, p)
            if on_top:
                kc = min(nc, kc + 1)
            if kept not in (count(n, kc, True), count(n, kc, False)):
                return False
        return True

    assert consistent(lambda nc, p: oracle.top_p_count(nc, p))
    assert not consistent(lambda nc, p: max(1, round(p * nc)))
    assert not consistent(lambda nc, p: max(1, math.floor(p * nc)))
    assert not consistent(lambda nc, p: oracle.top_p_count(nc, p), on_top=True)


@pytest.mark.parametrize("seed", range(5))
def test_selection_monotone_in_p_and_mass(seed):
    rng = np.random.default_rng(300 + seed)
    cs = rng.random(int(rng.integers(1, 300)))
    prev = None
    for p in np.linspace(0.01, 1.0, 40):
        cur = set(np.nonzero(oracle.select(cs, "top_p", p))[0])
        if prev is not None:
            assert prev <= cur
        prev = cur
    assert prev == set(range(cs.size))
    prev = None
    for m in np.linspace(0.01, 1.0, 40):
        cur = set(np.nonzero(oracle.select(cs, "mass", m))[0])
        if prev is not None:
            assert prev <= cur
        prev = cur


def test_select_single_chunk_and_bad_args():
    assert list(oracle.select([0.3], "top_p", 0.01)) == [1]
    assert list(oracle.select([0.3], "mass", 0.5)) == [1]
    with pytest.raises(ValueError):
        oracle.select([0.3, 0.1], "top_p", 0.0)
    with pytest.raises(ValueError):
        oracle.select([0.3, 0.1], "mass", 1.5)


# ----------------------------------------------------------------------------
# Compaction
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_gather_matches_list_comprehension(seed):
    rng = np.random.default_rng(400 + seed)
    n = int(rng.integers(1, 500))
    C = int(rng.choice([1, 7, 32]))
    nc = (n + C - 1) // C
    keep = (rng.random(nc) < 0.4).astype(np.uint8)
    ids = rng.integers(0, 1 << 17, n).astype(np.int32)
    ki, kp = oracle.gather(keep, ids, C)
    want = [t for t in range(n) if t == 0 or keep[t // C]]
    assert kp.tolist() == want
    assert ki.tolist() == [int(ids[t]) for t in want]
    assert ki.size == sum(min(C, n - c * C) for c in range(nc) if keep[c]) + (0 if keep[0] else 1)


# ----------------------------------------------------------------------------
# Whole path on small planted workloads
# ----------------------------------------------------------------------------

def test_planted_spans_selected_n800():
    """The 800-token fp32 workload (3 planted spans, top-p 0.15): all spans
    are kept and the kept count is 3 spans + the final chunk + BOS."""
    inp = workloads.make_inputs(workloads.WORKLOADS["n800_fp32"])
    out = oracle.pipeline(inp)
    keep = out["keep"][0]
    for c in inp.spans[0]:
        assert keep[c] == 1
    assert keep.sum() == oracle.top_p_count(25, 0.15) == 4
    assert out["kept_ids"][0].size == 3 * 32 + 32 + (0 if keep[0] else 1)


def test_planted_spans_selected_small_bf16_shapes():
    w = workloads.small_workload("n32k_bf16", lengths=(2500,), n_spans=6, seed=77)
    inp = workloads.make_inputs(w)
    for mode, param in (("mass", 0.85), ("top_p", 0.15)):
        out = oracle.pipeline(inp, mode, param)
        for c in inp.spans[0]:
            assert out["keep"][0][c] == 1, (mode, c)


def test_all_zero_q_gives_equal_chunk_scores():
    w = workloads.small_workload("n800_fp32", lengths=(300,))
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    out = oracle.pipeline(inp)
    cs = out["chunk_scores"][0]
    np.testing.assert_allclose(cs, cs[0], rtol=1e-13)


# ----------------------------------------------------------------------------
# Break-even gate (host arithmetic)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n, kept, want", [
    (600, 330, False),     # saves 270/270 = 1 s; scoring 600/600 = 1 s, x 1.2 = 1.2 s
    (600, 0, True),        # saves 600/270 = 2.2 s > 1.2 s
    (5400, 2700, False),   # saves 10 s; scoring 9 s, x 1.2 = 10.8 s
    (5400, 2000, True),    # saves 3400/270 = 12.6 s > 10.8 s
    (1, 1, False),         # nothing dropped
])
def test_break_even_hand_values(n, kept, want):
    assert oracle.break_even(n, kept) == want


def test_break_even_threshold_is_a_kept_fraction():
    """Both times grow with n, so with the default rates the gate only
    depends on the kept fraction f: run iff (1 - f) / 270 >= 1.2 / 600,
    i.e. f <= 0.46."""
    for n in (1000, 50000, 10 ** 7):
        assert oracle.break_even(n, int(0.45 * n))
        assert not oracle.break_even(n, int(0.47 * n))


# ----------------------------------------------------------------------------
# Standalone-tool semantics: window plan, stitching, legacy selection, thinning
# ----------------------------------------------------------------------------

def test_window_plan_worked_example_from_the_guide():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "window_plan_4471.txt"))
             if l.strip() and not l.startswith("#")]
    hdr = dict(zip(lines[0][0::2], map(int, lines[0][1::2])))
    want = [tuple(map(int, l)) for l in lines[1:]]
    plan = oracle.window_plan(hdr["n_tokens"], hdr["window"], hdr["stride"])
    got = [(s, s + n, s, s + k) for s, n, k in plan]
    assert got == want


@pytest.mark.parametrize("n, W, s", [(1, 2000, 1000), (999, 2000, 1000), (2000, 2000, 1000),
                                     (2001, 2000, 1000), (3000, 2000, 1000), (3001, 2000, 1000),
                                     (131072, 8192, 4096), (5000, 1000, 300), (777, 100, 100)])
def test_window_plan_covers_each_token_once_and_stops(n, W, s):
    plan = oracle.window_plan(n, W, s)
    cover = np.zeros(n, dtype=np.int64)
    for start, length, keep in plan:
        assert 1 <= keep <= length <= W and start + length <= n
        cover[start:start + keep] += 1
    assert np.all(cover == 1)
    # windows at 0, s, 2s, ... up to the first one that reaches the end
    assert len(plan) == max(0, -(-(n - W) // s)) + 1
    assert plan[-1][0] + plan[-1][1] == n


def test_stitch_averages_overlaps_and_defaults_to_one():
    plan = [(0, 4, 3), (2, 4, 2)]          # token 2 twice, token 5 never
    w0, w1 = [1.0, 2.0, 3.0, 9.0], [5.0, 7.0, 9.0, 9.0]
    got = oracle.stitch(plan, [w0, w1], 6)
    np.testing.assert_array_equal(got, [1.0, 2.0, 4.0, 7.0, 1.0, 1.0])


def test_stitch_of_a_v31_plan_is_a_plain_copy():
    plan = oracle.window_plan(4471, 2000, 1000)
    rng = np.random.default_rng(41)
    ws = [rng.random(n) for _, n, _ in plan]
    got = oracle.stitch(plan, ws, 4471)
    for (start, n, keep), w in zip(plan, ws):
        np.testing.assert_array_equal(got[start:start + keep], w[:keep])


def test_legacy_select_keeps_threshold_ties():
    scores = np.repeat([5.0, 5.0, 5.0, 1.0, 2.0], 32)          # 160 tokens, 5 chunks
    kept = oracle.select_legacy(scores, 32, 0.2, 4)           # kc = 1, threshold 5
    np.testing.assert_array_equal(kept, np.r_[0:96, 158, 159])


def test_legacy_select_always_tokens_and_min_fill():
    n = 1170                                                   # eff_min = 117
    scores = np.zeros(n)
    scores[320:352] = 1.0                                      # chunk 10 best
    scores[640:672] = 0.5                                      # chunk 20 second
    kept = oracle.select_legacy(scores, 32, 0.05, 128)         # nc 37, kc = ceil(1.85) = 2
    base = set(range(320, 352)) | set(range(640, 672)) | {0, 1, 2, 3, n - 2, n - 1}
    assert len(base) == 70
    fill = [t for t in range(n) if t not in base][:117 - 70]  # index order, low chunks first
    assert list(kept) == sorted(base | set(fill))
    assert len(kept) == 117


def test_legacy_select_keeps_everything_when_short_or_full():
    # the effective minimum is below n for every n > 4, so only n <= 4 keeps all
    np.testing.assert_array_equal(oracle.select_legacy(np.arange(4.0), 32, 0.3, 128), np.arange(4))
    np.testing.assert_array_equal(oracle.select_legacy(np.arange(3.0), 32, 0.3, 128), np.arange(3))
    # n = 40: the tail chunk (tokens 32-39, the larger mean) plus tokens 0-3
    np.testing.assert_array_equal(oracle.select_legacy(np.arange(40.0), 32, 0.01, 128),
                                  np.r_[0:4, 32:40])
    np.testing.assert_array_equal(oracle.select_legacy(np.arange(500.0), 32, 1.0, 128),
                                  np.arange(500))


@pytest.mark.parametrize("seed", range(8))
def test_legacy_select_matches_rank_formulation(seed):
    """Independent route: a chunk is in iff fewer than kc chunk means are
    strictly larger (same as reaching the kc-th largest, ties included)."""
    rng = np.random.default_rng(50 + seed)
    n = int(rng.integers(200, 3000))
    C = int(rng.choice([16, 32, 64]))
    scores = np.round(rng.random(n) * 4) / 4                   # many ties
    p = float(rng.choice([0.1, 0.3, 0.5]))
    kept = set(oracle.select_legacy(scores, C, p, 10 ** 9 if seed % 2 else 4).tolist())
    nc = -(-n // C)
    means = np.array([np.float32(scores[c * C:(c + 1) * C].mean()) for c in range(nc)])
    kc = oracle.legacy_keep_count(nc, p)
    chunk_in = [(means > means[c]).sum() < kc for c in range(nc)]
    want = {t for c in range(nc) if chunk_in[c] for t in range(c * C, min(n, (c + 1) * C))}
    want |= {0, 1, 2, 3, n - 2, n - 1}
    eff_min = min(10 ** 9 if seed % 2 else 4, max(4, n // 10))
    rest = [t for t in range(n) if t not in want]
    want |= set(rest[:max(0, eff_min - len(want))])
    assert kept == want


def test_legacy_keep_count_is_single_precision():
    assert oracle.legacy_keep_count(37, 0.3) == 12
    assert oracle.legacy_keep_count(1, 0.01) == 1
    # float32(0.7) * 10 rounds to 7.0000000 in single precision: no ceil to 8
    assert oracle.legacy_keep_count(10, 0.7) == 7


def test_thin_hand_values():
    np.testing.assert_array_equal(oracle.thin(np.arange(10), 3), [0, 3, 9])
    np.testing.assert_array_equal(oracle.thin(np.arange(7), 3), [0, 2, 6])
    np.testing.assert_array_equal(oracle.thin(np.arange(5), 5), np.arange(5))
    k = np.arange(0, 20000, 3)
    out = oracle.thin(k, 2000)                                 # step 3
    assert out.size == 2000 and out[-1] == k[-1] and np.all(out[:-1] == k[:3 * 1999:3])
