"""CPU checks of the bf16 output-norm bar (tests/gated_bound.py): an exact
output passes, an error beyond the derived bound fails, rows below the bar
are checked against the GPU's own recurrence output and held to the stated
fraction."""
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
    ex, nex = check_norm_bound(y_ref.copy(), y_ref, ot, s, 1e-2, eps, ot)
    assert ex == 0.0 and nex == 0


def test_error_beyond_bound_fails():
    ot, s, eps, y_ref = _case()
    y = y_ref.copy()
    y[3, 5] += 0.5          # far beyond s E (1 + |o~|/r) / (r - E) for an O(1) row
    with pytest.raises(AssertionError):
        check_norm_bound(y, y_ref, ot, s, 1e-2, eps, ot)


def test_recurrence_output_is_held_to_the_plain_bar():
    ot, s, eps, y_ref = _case()
    bad = ot.copy()
    bad[0, 0] += 0.05 * np.max(np.abs(ot))
    with pytest.raises(AssertionError):
        check_norm_bound(y_ref.copy(), y_ref, ot, s, 1e-2, eps, bad)


def test_rows_below_the_bar_are_checked_against_their_own_output_step():
    ot, s, eps, y_ref = _case()
    ot[7] *= 1e-5           # r_ref far below E = 1e-2 max|o~|
    y_ref[7] = s[7] * ot[7] / np.sqrt(np.mean(ot[7] ** 2) + eps)
    # the GPU's recurrence output for that row may differ from the reference
    # by up to E (here: a different direction altogether) ...
    og = ot.copy()
    og[7] = 1e-3 * np.roll(ot[7] / np.max(np.abs(ot[7])), 3)
    y = y_ref.copy()
    y[7] = s[7] * og[7] / np.sqrt(np.mean(og[7] ** 2) + eps)
    ex, nex = check_norm_bound(y, y_ref, ot, s, 1e-2, eps, og)
    assert nex == 1
    # ... but y must follow it through the output step
    y[7, 2] *= 1.1
    with pytest.raises(AssertionError):
        check_norm_bound(y, y_ref, ot, s, 1e-2, eps, og)


def test_too_many_rows_below_the_bar_fail():
    ot, s, eps, y_ref = _case()
    n = int(MAX_EXEMPT_FRACTION * ot.shape[0]) + 1
    ot[:n] *= 1e-6
    y_ref[:n] = s[:n] * ot[:n] / np.sqrt(np.mean(ot[:n] ** 2, -1, keepdims=True) + eps)
    with pytest.raises(AssertionError):
        check_norm_bound(y_ref.copy(), y_ref, ot, s, 1e-2, eps, ot)
