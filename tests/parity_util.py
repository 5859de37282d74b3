"""Comparison helpers for the GPU parity tests (plain numpy; no method arithmetic here)."""

import numpy as np

# Tolerances fixed by the method's acceptance bar: fp32 outputs within 1e-5 relative (read per
# (query, head) vector: max |diff| <= 1e-5 * max |reference|), bf16 / fp8 outputs within 2e-2
# absolute on unit-variance inputs (max over all elements).
FP32_REL = 1e-5
BF16_ABS = 2e-2


def assert_fp32_close(got, want, rel=FP32_REL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max(axis=-1)
    ref = np.abs(want).max(axis=-1)
    bad = err > rel * ref
    assert not bad.any(), f"fp32 parity: worst ratio {np.max(err / np.maximum(ref, 1e-300)):.3e}"


def assert_abs_close(got, want, tol=BF16_ABS):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max()
    assert err <= tol, f"abs parity: max |diff| {err:.4e} > {tol}"


def topk_delta(q_idx, w, keys):
    """Conservative bound on fp32 accumulation error of any one indexer score:
    2^-20 * max_g sum_h |w_h| sum_d |q_hd k_gd|."""
    if keys.shape[0] == 0:
        return 0.0
    mag = np.abs(w)[:, None] * (np.abs(q_idx) @ np.abs(keys).T)
    return float(2.0 ** -20 * mag.sum(axis=0).max())


def check_topk_set(got_row, want_row, scores, delta, k):
    """Sets must be equal unless the difference lies within delta of the k-th score.
    Returns the number of near-tie swaps (0 when the sets are identical)."""
    got = [int(g) for g in got_row if g >= 0]
    want = [int(g) for g in want_row if g >= 0]
    assert got == sorted(got), "output not ascending"
    assert len(set(got)) == len(got), "duplicate index"
    assert len(got) == len(want), f"selected {len(got)} != {len(want)}"
    assert all(g < len(scores) for g in got), "index outside the visible range"
    pad = list(got_row[len(got):])
    assert all(int(v) == -1 for v in pad), "padding must be -1"
    diff = set(got) ^ set(want)
    if not diff:
        return 0
    kth = np.sort(scores)[::-1][min(k, len(scores)) - 1]
    far = [g for g in diff if abs(scores[g] - kth) > delta]
    assert not far, f"top-k differs beyond the fp32 bound at {far[:5]} (delta {delta:.3e})"
    return len(diff) // 2
