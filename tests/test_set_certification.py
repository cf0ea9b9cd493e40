"""The certified comparison of look-ahead index sets (tests/gpu_helpers.py) on the
CPU: differences explained by the per-index rounding bounds pass, others fail.

The GPU computes its own predictor scores, so its top-k may differ from the
oracle's at the threshold; the checker must accept exactly the differences the
certified bounds allow and reject a set that drops or adds an index the bounds
rule out.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import check_sets_certified


def _scores(B=3, N=200, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, N))


def test_identical_sets_pass():
    s = _scores()
    from oracle import dv_oracle as O
    ref = O.select_sets(s.astype(np.float32).astype(np.float64), 20, True)
    assert check_sets_certified(ref, s, 20, True, np.full_like(s, 1e-6), "same") == 0


def test_swap_within_bounds_passes():
    s = _scores(B=1)
    k = 20
    order = np.argsort(-s[0], kind="stable")
    kth, nxt = order[k - 1], order[k]          # the k-th and the (k+1)-th index
    # a GPU that swapped them: legal if their bounds overlap
    gap = s[0, kth] - s[0, nxt]
    bound = np.full_like(s, 0.6 * gap)
    got = np.sort(np.append(order[: k - 1], nxt))
    assert check_sets_certified(got, s, k, True, bound, "swap") == 2


def test_swap_outside_bounds_fails():
    s = _scores(B=1)
    k = 20
    order = np.argsort(-s[0], kind="stable")
    kth, nxt = order[k - 1], order[k]
    gap = s[0, kth] - s[0, nxt]
    bound = np.full_like(s, 0.4 * gap)          # bounds do not overlap
    got = np.sort(np.append(order[: k - 1], nxt))
    with pytest.raises(AssertionError):
        check_sets_certified(got, s, k, True, bound, "swap")


def test_per_index_bound_not_row_max():
    """One index with a huge bound elsewhere in the row must not certify a swap
    between two indices whose own bounds are tiny."""
    s = _scores(B=1, N=300, seed=4)
    k = 30
    order = np.argsort(-s[0], kind="stable")
    kth, far = order[k - 1], order[k + 5]       # a swap reaching 6 places down
    bound = np.full_like(s, 1e-9)
    bound[0, order[-1]] = 1e3                   # the row maximum is huge
    got = np.sort(np.append(order[: k - 1], far))
    with pytest.raises(AssertionError):
        check_sets_certified(got, s, k, True, bound, "row max")


def test_union_difference_needs_every_row():
    """In a union, an index the oracle took in row 0 may be left out by the GPU only
    if row 0's bounds allow it."""
    s = _scores(B=2, N=100, seed=7)
    k = 10
    from oracle import dv_oracle as O
    ref = O.select_sets(s.astype(np.float32).astype(np.float64), k, True)
    top0 = np.argsort(-s[0], kind="stable")[:k]
    top1 = np.argsort(-s[1], kind="stable")[:k]
    only0 = np.setdiff1d(top0, top1)
    drop = only0[np.argmax(s[0, only0])]        # the best-ranked index unique to row 0
    got = np.setdiff1d(ref, [drop])
    with pytest.raises(AssertionError):
        check_sets_certified(got, s, k, True, np.full_like(s, 1e-9), "union")
