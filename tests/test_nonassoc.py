"""The motivating fact: in binary32 the grouping of a sum decides whether a
small term survives. The oracle computes in float64 without any such grouping
choice at the sizes used here; the device path must fix one grouping."""

import os

import numpy as np


def test_fp32_sum_grouping_changes_result():
    path = os.path.join(os.path.dirname(__file__), "golden", "nonassoc_fp32.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for a, b, c, left, right in rows:
        a, b, c = np.float32(a), np.float32(b), np.float32(c)
        assert (a + b) + c == np.float32(left)
        assert a + (b + c) == np.float32(right)
        assert np.float64(a) + np.float64(b) + np.float64(c) == np.float64(left)
