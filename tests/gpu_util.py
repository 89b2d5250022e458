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
