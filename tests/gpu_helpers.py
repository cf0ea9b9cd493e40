"""Helpers shared by the GPU parity tests: host views of device tensors for the
oracle, tolerance checks, and the certified comparison of index sets."""
from __future__ import annotations

import numpy as np
import torch

from oracle import dv_oracle as O

U32 = 2.0 ** -24   # unit roundoff of fp32

# Tolerances relative to max|ref| (the oracle's float64 result).
#  * BOUND_* is the acceptance bound of the method's parity goal: 1e-5 for fp32
#    weights, 2e-2 for bf16 weights with fp32 accumulation.
#  * TIGHT_* is a sharper bound from the arithmetic: inputs are exact for both
#    sides, so the only difference is fp32 rounding.  A dot product of K terms
#    computed in fp32 typically errs by about sqrt(K) * u relative to the sum of
#    |terms|; for K <= 50k that is below 1e-5 of max|ref|, and 2e-4 leaves a wide
#    margin while still failing on one dropped or doubled row of W1/W2 (each row
#    moves the output by about 1/sqrt(|S|) of max|ref|, > 4e-3 at |S| <= 50k).
#    Attention adds the conditioning of exp at large logits: an absolute logit
#    error e turns into a relative weight error e; with |logit| up to ~100 and
#    fp32 logits good to ~1e-5 relative this is ~1e-3, hence 5e-3 there.
BOUND_F32, BOUND_BF16 = 1e-5, 2e-2
TIGHT_MLP, TIGHT_ATTN = 2e-4, 5e-3


def banner(msg: str):
    """Name the case on stderr before a GPU step (a fault may end the process)."""
    import sys
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Host copy of a stored tensor in the oracle's conventions (bf16 -> uint16 bits)."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    if scale == 0.0:
        return err
    return err / scale


def assert_close(got, ref, tol, what=""):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite output"
    assert e <= tol, f"{what}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def score_bound(y, A, Bm) -> np.ndarray:
    """Certified bound on |fp32 score - exact score| for s = (y A) B computed as two
    fp32 dot products of lengths d and r (any summation order):
        |err_j| <= g * ( sum_t |z_t||B_tj| + sum_t |B_tj| sum_i |y_i||A_ti| ),
    g = 2 (d + r) u, u = 2^-24.  Returns [B][N]."""
    y = O.widen(y)
    A = O.widen(A)
    Bm = O.widen(Bm)
    d, r = y.shape[1], A.shape[0]
    g = 2.0 * (d + r) * U32
    z = np.abs(y @ A.T)
    za = np.abs(y) @ np.abs(A).T
    return g * ((z + za) @ np.abs(Bm))


def check_sets_certified(got, ref_scores, k, union, bound, what=""):
    """GPU union index set vs the oracle's, allowing only differences that the
    certified per-index rounding bounds explain.

    ``ref_scores`` are the oracle's float64 scores [B][N] and ``bound`` their
    certified error [B][N] (``score_bound``).  With eps_j = bound_j plus two units of
    fp32 rounding of s_j, every GPU score lies in [lo_j, hi_j] = [s_j - eps_j,
    s_j + eps_j].  Then, row by row:
      * an index j the GPU took but the oracle did not must be one that some row's
        GPU top-k could hold: fewer than k indices i of that row have lo_i > hi_j
        (those certainly rank above j on the GPU);
      * an index j the oracle took (in row b's top-k) but the GPU left out of every
        row must be one the GPU could rank below k others in each such row b: at
        least k indices i != j have hi_i >= lo_j.
    Both conditions follow from the bounds alone (no tolerance is assumed), and
    they certify each differing index through its own and its rivals' bounds.
    Returns the number of differing indices."""
    assert union, "the decode layer's look-ahead sets are unions"
    s32 = ref_scores.astype(np.float32).astype(np.float64)
    per_row = O.select_sets(s32, k, False)
    ref_set = O.select_sets(s32, k, True)
    got = np.asarray(got, dtype=np.int64)
    assert np.all(np.diff(got) > 0), f"{what}: set not strictly ascending"
    took = np.setdiff1d(got, ref_set)       # GPU took, oracle did not
    left = np.setdiff1d(ref_set, got)       # oracle took, GPU did not
    if took.size == 0 and left.size == 0:
        return 0
    s = np.asarray(ref_scores, dtype=np.float64)
    eps = np.asarray(bound, dtype=np.float64) + 2.0 * U32 * np.abs(s)
    lo, hi = s - eps, s + eps
    B = s.shape[0]
    lo_sorted = [np.sort(lo[b]) for b in range(B)]
    hi_sorted = [np.sort(hi[b]) for b in range(B)]
    for j in took:
        # number of indices certainly above j in row b
        above = [lo_sorted[b].size - np.searchsorted(lo_sorted[b], hi[b, j], side="right")
                 for b in range(B)]
        assert min(above) < k, (f"{what}: index {j} is in the GPU set, but in every row at "
                                f"least k = {k} indices certainly outrank it")
    for j in left:
        for b in range(B):
            if j not in per_row[b]:
                continue
            # indices other than j that may rank above j in row b
            maybe = hi_sorted[b].size - np.searchsorted(hi_sorted[b], lo[b, j], side="left") - 1
            assert maybe >= k, (f"{what}: index {j} is in the oracle's row-{b} top-{k}, which "
                                f"the GPU could not have left: only {maybe} rivals may outrank it")
    return int(took.size + left.size)
