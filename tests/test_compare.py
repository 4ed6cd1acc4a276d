"""The byte comparator used by every bitwise test can fail (no GPU)."""

import numpy as np

from tests.helpers import bitwise_report, diff_stats


def test_comparator_detects_one_ulp():
    a = np.linspace(-20, 0, 1000).astype(np.float32)
    b = a.copy()
    b.view(np.uint32)[123] ^= 1
    r = bitwise_report(a, b)
    assert r["mismatch_count"] == 1 and r["max_abs_diff"] > 0
    assert bitwise_report(a, a.copy()) == {"mismatch_count": 0, "max_abs_diff": 0.0}


def test_comparator_separates_signed_zero_and_nan_payloads():
    a = np.array([0.0, 1.0], np.float32)
    b = np.array([-0.0, 1.0], np.float32)
    assert bitwise_report(a, b)["mismatch_count"] == 1
    n = np.array([np.nan], np.float32)
    assert bitwise_report(n, n.copy())["mismatch_count"] == 0


def test_diff_stats():
    s = diff_stats(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.5, 3.0]), np.array([True, True, False]))
    assert s["max"] == 0.5 and s["n"] == 2
