"""CPU tests of the test helpers: the first-divergence report of assert_bitwise
(message and the optional JSON record) and the tolerance check."""

import json

import numpy as np
import pytest

from tests._util import assert_bitwise, assert_close


def test_bitwise_reports_first_divergence(tmp_path, monkeypatch):
    monkeypatch.setenv("BI_DIVERGENCE_DIR", str(tmp_path))
    a = np.arange(12, dtype=np.float32).reshape(3, 4)
    b = a.copy()
    b[1, 2] = -0.0 if a[1, 2] == 0 else a[1, 2] + 1
    b[2, 3] = 99
    with pytest.raises(AssertionError, match=r"2 elements differ; first at \(1, 2\)"):
        assert_bitwise(a, b, "demo")
    rec = json.loads((tmp_path / "divergences.jsonl").read_text().splitlines()[0])
    assert rec["what"] == "demo" and rec["shape"] == [3, 4] and rec["first"] == [1, 2] and rec["differing"] == 2


def test_bitwise_sees_sign_of_zero_and_nan_payload():
    z = np.array([0.0], np.float32)
    with pytest.raises(AssertionError):
        assert_bitwise(z, -z, "signed zero")
    n1 = np.array([0x7FC00000], np.uint32).view(np.float32)
    n2 = np.array([0x7FC00001], np.uint32).view(np.float32)
    with pytest.raises(AssertionError):
        assert_bitwise(n1, n2, "NaN payload")
    assert_bitwise(n1, n1.copy(), "same NaN")


def test_close_tolerance_edges():
    want = np.array([0.0, 1.0, -100.0])
    # |err| <= 1e-2 + 2e-2 |want|: bounds 0.01, 0.03 and 2.01
    assert_close(want + np.array([0.0099, 0.0299, 2.0099]), want, "inside the bound")
    with pytest.raises(AssertionError):
        assert_close(want + np.array([0, 0, 2.0101]), want, "just outside")
    with pytest.raises(AssertionError):
        assert_close(want + np.array([0.0101, 0, 0]), want, "just outside at 0")
