"""The CPU oracle against facts outside itself (hand-worked examples, library
routines for the dense cases, invariants, closed forms, brute force)."""
import pytest

import pins
from oracle import dv_oracle


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(dv_oracle)


def test_oracle_rejects_nonfinite_scores():
    import numpy as np
    with pytest.raises(ValueError):
        dv_oracle.topk_row(np.array([1.0, np.nan, 2.0]), 1)
