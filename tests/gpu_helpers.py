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
    """GPU index set vs the oracle's, allowing only swaps certified by rounding.

    `ref_scores` are the oracle's float64 scores [B][N] and `bound` their certified
    error [B][N].  Every index in the symmetric difference of the GPU set and the
    oracle set must lie within bound of the k-th score of some row."""
    ref_set = O.select_sets(ref_scores.astype(np.float32).astype(np.float64), k, union)
    got = np.asarray(got, dtype=np.int64)
    assert np.all(np.diff(got) > 0), f"{what}: set not strictly ascending"
    diff = np.setxor1d(got, ref_set)
    if diff.size == 0:
        return 0
    B, N = ref_scores.shape
    kth = [np.sort(ref_scores[b])[::-1][min(k, N) - 1] if k > 0 else np.inf for b in range(B)]
    for j in diff:
        ok = False
        for b in range(B):
            # a swap needs two scores that straddle the k-th one and move past each
            # other: both lie within the sum of two certified bounds of it
            tol = 2.0 * float(bound[b].max()) + 4.0 * U32 * abs(kth[b])
            if abs(ref_scores[b, j] - kth[b]) <= tol:
                ok = True
                break
        assert ok, f"{what}: index {j} differs from the oracle set and is not borderline"
    return int(diff.size)
