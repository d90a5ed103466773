"""Comparison helpers for the GPU parity tests (no GPU needed to import).

Tolerances:
* importance, token and chunk scores: rel 1e-3, abs 1e-6 against the fp64
  oracle (the GPU accumulates in fp32);
* kept chunks: identical, except chunks whose oracle score lies within 1e-5
  of the oracle's selection cutoff (the score of the last chunk its walk
  admitted); in mass mode also the chunk after the crossing one when the
  oracle's running sum ends within 1e-6 * total of the threshold;
* kept ids, positions and offsets: identical (integers). Where kept chunks
  differ by an excused chunk, the GPU's compaction is instead checked
  exactly against the oracle's compaction of the GPU's own keep flags.
* the selection rule itself: the oracle's rule applied to the GPU's own chunk
  scores must give the GPU's keep flags, except where the two precisions may
  legitimately disagree: the kernel orders scores by 32-bit fixed point
  relative to the prompt's largest score (ties by index) and sums them in
  64-bit fixed point, the oracle orders by value and sums in fp64. Excused
  are chunks within 2^-31 of the largest score from the cutoff and, in mass
  mode, the chunks around a crossing whose running sum lies within 1e-9 of
  the total from the threshold.
"""
import numpy as np

import oracle

RTOL, ATOL, CUTOFF_TOL, MASS_TOL = 1e-3, 1e-6, 1e-5, 1e-6
KEY_TOL, SUM_TOL = 2.0 ** -31, 1e-9     # precision of the kernel's selection arithmetic


def assert_scores_close(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bad = np.abs(got - want) > ATOL + RTOL * np.abs(want)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside rel {RTOL} / abs "
                             f"{ATOL}; first at {i}: got {got[i]!r} want {want[i]!r}")


def excused_chunks(ora_cs, ora_keep, mode, param, cutoff_tol=CUTOFF_TOL, mass_tol=MASS_TOL):
    """Set of chunk indices whose keep decision may differ from the oracle's."""
    cs = np.asarray(ora_cs, dtype=np.float64)
    nc = cs.size
    kept = [i for i in np.flatnonzero(ora_keep) if i != nc - 1]
    excused = set()
    if kept:
        cutoff = cs[kept].min()
        excused |= set(int(i) for i in np.flatnonzero(np.abs(cs - cutoff) <= cutoff_tol))
    if mode == "mass" and nc > 1:
        order = sorted(range(nc - 1), key=lambda i: (-cs[i], i))
        total = cs.sum()
        target = param * total
        cum = cs[nc - 1]
        for pos, i in enumerate(order):
            if abs(cum - target) <= mass_tol * total:
                excused.add(int(i))                      # first chunk the walk may or may not take
                if pos > 0:
                    excused.add(int(order[pos - 1]))
            if cum >= target:
                break
            cum += cs[i]
    excused.discard(nc - 1)
    return excused


def check_prompt(gpu, ora, b, mode, param, C, ids):
    """Compare one prompt's chunk scores, keep flags and compaction.

    gpu: dict with per-prompt numpy arrays 'chunk_scores', 'keep',
    'kept_ids', 'kept_pos'. Returns the number of excused differing chunks.
    """
    assert_scores_close(gpu["chunk_scores"], ora["chunk_scores"][b], f"chunk scores, prompt {b}")
    # Selection logic in the same precision: the oracle's rule applied to the
    # GPU's own chunk scores must give the GPU's keep flags exactly.
    own_cs = np.asarray(gpu["chunk_scores"], dtype=np.float64)
    own = oracle.select(own_cs, mode, param)
    own_diff = np.flatnonzero(gpu["keep"] != own)
    if own_diff.size:
        ex = excused_chunks(own_cs, own, mode, param, cutoff_tol=KEY_TOL * own_cs.max(),
                            mass_tol=SUM_TOL)
        bad = [int(i) for i in own_diff if int(i) not in ex]
        assert not bad, f"prompt {b}: selection differs on the GPU's own scores at {bad[:10]}"
    diff = np.flatnonzero(gpu["keep"] != ora["keep"][b])
    if diff.size:
        ex = excused_chunks(ora["chunk_scores"][b], ora["keep"][b], mode, param)
        unexcused = [int(i) for i in diff if int(i) not in ex]
        assert not unexcused, f"prompt {b}: kept chunks differ at {unexcused[:10]}"
    want_ids, want_pos = oracle.gather(gpu["keep"], ids, C)
    assert np.array_equal(gpu["kept_pos"], want_pos), f"prompt {b}: kept positions differ"
    assert np.array_equal(gpu["kept_ids"], want_ids), f"prompt {b}: kept ids differ"
    if not diff.size:
        assert np.array_equal(gpu["kept_pos"], ora["kept_pos"][b])
        assert np.array_equal(gpu["kept_ids"], ora["kept_ids"][b])
    return int(diff.size)
