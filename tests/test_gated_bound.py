"""CPU checks of the bf16 output-norm bar (tests/gated_bound.py): an exact
output passes, an error beyond the derived bound fails, rows below the bar
are counted and held to their cap and to the stated fraction."""
import numpy as np
import pytest

from gated_bound import MAX_EXEMPT_FRACTION, check_norm_bound


def _case(rows=400, dv=16, seed=0):
    rng = np.random.default_rng(seed)
    ot = rng.standard_normal((rows, dv))
    s = 1.0 / (1.0 + np.exp(-rng.standard_normal((rows, dv))))
    eps = 1e-6
    y_ref = s * ot / np.sqrt(np.mean(ot * ot, -1, keepdims=True) + eps)
    return ot, s, eps, y_ref


def test_exact_output_passes_and_counts_nothing():
    ot, s, eps, y_ref = _case()
    ex, nex = check_norm_bound(y_ref.copy(), y_ref, ot, s, 1e-2, eps)
    assert ex == 0.0 and nex == 0


def test_error_beyond_bound_fails():
    ot, s, eps, y_ref = _case()
    y = y_ref.copy()
    y[3, 5] += 0.5          # far beyond s E (1 + |o~|/r) / (r - E) for an O(1) row
    with pytest.raises(AssertionError):
        check_norm_bound(y, y_ref, ot, s, 1e-2, eps)


def test_rows_below_the_bar_are_counted_and_capped():
    ot, s, eps, y_ref = _case()
    ot[7] *= 1e-5           # r_ref far below E = 1e-2 max|o~|
    y_ref[7] = s[7] * ot[7] / np.sqrt(np.mean(ot[7] ** 2) + eps)
    y = y_ref.copy()
    y[7] = -y[7]            # any value within the cap is accepted for such a row
    ex, nex = check_norm_bound(y, y_ref, ot, s, 1e-2, eps)
    assert nex == 1
    y[7, 0] = 2.0 * np.sqrt(ot.shape[1])  # beyond |s| sqrt(dv)
    with pytest.raises(AssertionError):
        check_norm_bound(y, y_ref, ot, s, 1e-2, eps)


def test_too_many_rows_below_the_bar_fail():
    ot, s, eps, y_ref = _case()
    n = int(MAX_EXEMPT_FRACTION * ot.shape[0]) + 1
    ot[:n] *= 1e-6
    y_ref[:n] = s[:n] * ot[:n] / np.sqrt(np.mean(ot[:n] ** 2, -1, keepdims=True) + eps)
    with pytest.raises(AssertionError):
        check_norm_bound(y_ref.copy(), y_ref, ot, s, 1e-2, eps)
