"""The parity bar itself: two separate bounds (max abs 2e-3, max rel 1e-2), not one combined."""
import numpy as np

from tests.helpers import tolerance_report


def test_absolute_bound_alone_fails():
    ref = np.array([0.5, 1.0, 2.0])
    ok, ma, _ = tolerance_report(ref + np.array([0.0, 0.0, 2.5e-3]), ref)
    assert not ok and abs(ma - 2.5e-3) < 1e-12        # rel 1.25e-3 passes, abs 2.5e-3 does not


def test_relative_bound_alone_fails():
    ref = np.array([0.01, 0.3, -0.2])
    got = ref + np.array([2e-4, 0.0, 0.0])             # abs 2e-4 passes, rel 2e-2 does not
    ok, ma, mr = tolerance_report(got, ref)
    assert not ok and abs(mr - 2e-2) < 1e-9
    # the combined form |g - r| <= 2e-3 + 1e-2 |r| would have passed it
    assert np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref))


def test_tiny_references_only_count_absolutely():
    ref = np.array([1e-6, -5e-4, 0.0])
    ok, _, mr = tolerance_report(ref + 1e-5, ref)
    assert ok and mr == 0.0


def test_non_finite_fails():
    assert not tolerance_report(np.array([np.nan]), np.array([0.0]))[0]
    assert not tolerance_report(np.array([np.inf]), np.array([1.0]))[0]


def test_within_both_bounds_passes():
    ref = np.linspace(-1, 1, 101)
    ok, ma, mr = tolerance_report(ref * (1 + 1e-3), ref)
    assert ok and ma <= 1.0001e-3 and mr <= 1.0001e-3
