"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

from __future__ import annotations

import sys

import numpy as np

BF16_STEP_REL = 2.0 ** -7     # one bf16 step (ulp) is at most 2^-7 |x|
BF16_HALF_STEP_REL = 2.0 ** -8


def say(*a):
    """Print and flush before a GPU step so a failing run names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tol(ref: np.ndarray, atol: float = 1e-2, rel: float = BF16_HALF_STEP_REL) -> np.ndarray:
    return atol + rel * np.abs(ref)


def assert_close_bf16(got, ref, atol=1e-2, rel=BF16_HALF_STEP_REL, what=""):
    """|g - r| <= atol + rel |r| elementwise.

    Against an unrounded reference a bf16 store adds at most half a step
    (rel = 2^-8).  Two stored values rounded independently from nearly equal
    inputs can differ by one step per storage rounding on the way
    (rel = n * 2^-7)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    tol = bf16_tol(ref, atol, rel)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def assert_close_bf16_rotated(got, ref, atol=1e-2, what=""):
    """Keys [..., d] that went through two bf16 stores with a RoPE rotation
    between them (the segment cache, then the realigned copy).

    The rotation mixes the two halves of each pair (e, e + d/2): a one-step
    difference in the first store of one component reaches the other
    component scaled by the sine, so the bound is relative to the pair's
    norm n_e (unchanged by the rotation): |g - r| <= atol + 2^-7 sqrt(2) n_e
    (first store) + 2^-8 |r| (second store)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    h = ref.shape[-1] // 2
    norm = np.sqrt(ref[..., :h] ** 2 + ref[..., h:] ** 2)
    norm = np.concatenate([norm, norm], axis=-1)
    tol = atol + BF16_STEP_REL * np.sqrt(2.0) * norm + BF16_HALF_STEP_REL * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def assert_close_f32(got, ref, rel=1e-4, what=""):
    """fp32 storage: max |g - r| <= rel * max |r| per tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = max(np.max(np.abs(ref)), 1e-30)
    err = np.max(np.abs(got - ref))
    assert err <= rel * scale, f"{what}: max err {err:.3g} > {rel} * {scale:.3g}"
    return float(err / scale)


def bf16_ulps(a, b) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16-representable values."""
    def key(x):
        x = np.asarray(x, dtype=np.float32)
        u = (x.view(np.uint32) >> 16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def selection_contract(gpu_sel, ora_scores, cand, k, tol):
    """Top-k parity under floating-point scores: identical sets whenever the
    oracle's k-th/(k+1)-th margin exceeds 2*tol; otherwise differences only
    among candidates whose oracle score is within 2*tol of the k-th score.
    Returns the number of differing indices."""
    import oracle
    ref = oracle.select_topk(ora_scores, cand, k)
    got = np.sort(np.asarray(gpu_sel, dtype=np.int64))
    assert len(got) == k and np.all(np.diff(got) > 0)
    assert np.all(np.isin(got, cand))
    if k == 0 or k == len(cand):
        assert np.array_equal(got, ref)
        return 0
    s = np.sort(ora_scores[cand])[::-1]
    kth, nxt = s[k - 1], s[k]
    diff = np.setxor1d(got, ref)
    if kth - nxt > 2 * tol:
        assert len(diff) == 0, f"selection differs with margin {kth - nxt:.3g} > 2*tol {2 * tol:.3g}"
    else:
        near = np.abs(ora_scores[diff] - kth) <= 2 * tol
        assert near.all(), "selection differs outside the near-tie band"
    return len(diff)


O_STRICT_LIMIT = 2.56   # below this |r|, a bf16 store's half step is under 1e-2


def assert_o_bf16(got, ref, what=""):
    """Layer output against the unrounded oracle: max |g - r| <= 1e-2 wherever
    |r| < 2.56 (the bound the output contract states; a bf16 store of such a
    value is off by at most 2^-8 |r| < 1e-2), and 1e-2 + 2^-8 |r| for larger
    |r|, where the store alone can exceed 1e-2.  Returns the max abs error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    small = np.abs(ref) < O_STRICT_LIMIT
    tol = np.where(small, 1e-2, 1e-2 + BF16_HALF_STEP_REL * np.abs(ref))
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


SCORE_REL_TOL = 1e-5    # GPU scores vs oracle scores from the GPU's own Q and K


def check_selection(gpu_scores, gpu_sel, ref_scores, cand, k, what=""):
    """Index parity of the Sparse-Q selection.

    ref_scores are the oracle's attention-mass scores computed from the
    query and key values the GPU stored (so storage rounding is not part of
    the comparison).  Checks, in order:
      1. the GPU's selection is exactly the top-k of the GPU's own scores
         (score descending, lower index first);
      2. every score is within 1e-5 * max(ref) of the oracle's;
      3. the selection equals the oracle's top-k on ref_scores, except for
         indices whose oracle score lies within 2 * tol of the k-th one,
         where scores equal within tolerance may order either way; with a
         k-th/(k+1)-th margin above 2 * tol there may be no difference.
    Returns (number of differing indices, max score error / max ref)."""
    import oracle
    gpu_scores = np.asarray(gpu_scores, dtype=np.float64)
    ref_scores = np.asarray(ref_scores, dtype=np.float64)
    cand = np.asarray(cand, dtype=np.int64)
    got = np.sort(np.asarray(gpu_sel, dtype=np.int64))
    assert np.array_equal(got, oracle.select_topk(gpu_scores, cand, k)), \
        f"{what}: selection is not the top-k of the GPU's own scores"
    smax = float(np.max(ref_scores[cand])) if len(cand) else 0.0
    tol = SCORE_REL_TOL * max(smax, 1e-30)
    err = float(np.max(np.abs(gpu_scores[cand] - ref_scores[cand]))) if len(cand) else 0.0
    assert err <= tol, f"{what}: score error {err:.3g} > {SCORE_REL_TOL} * max {smax:.3g}"
    nd = selection_contract(got, ref_scores, cand, k, tol)
    if 0 < k < len(cand):
        s = np.sort(ref_scores[cand])[::-1]
        band = int(np.sum(np.abs(ref_scores[cand] - s[k - 1]) <= 2 * tol))
        assert nd <= 2 * band, f"{what}: {nd} differences for {band} candidates in the near-tie band"
    return nd, err / max(smax, 1e-30)


def probe_lse_and_scores(q_sq, sq_pos, K):
    """Oracle LSE and attention-mass scores of the Sparse-Q rows from given
    (GPU-stored) queries and keys."""
    import oracle
    _, lse = oracle.causal_attention(q_sq, sq_pos, K, K)
    return lse, oracle.attention_mass_scores(q_sq, sq_pos, K, lse)
