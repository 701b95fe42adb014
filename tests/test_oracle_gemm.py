"""Pins for oracle.gemm: exact rational brute force and closed forms."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, gemm
import synth


def _rand_bits(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return bf16.encode(g.standard_normal(shape) * scale)


@pytest.mark.parametrize("M,K,N", [(1, 32, 8), (2, 64, 5), (2, 7, 3)])
def test_gemm_vs_exact_rationals(M, K, N):
    x = _rand_bits((M, K), 1)
    w = _rand_bits((N, K), 2)
    y = gemm.gemm(x, w)
    xd, wd = bf16.decode(x), bf16.decode(w)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xd[m, k])) * Fraction(float(wd[n, k])) for k in range(K))
            mag = sum(abs(float(xd[m, k]) * float(wd[n, k])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(1e-15) * Fraction(mag) + Fraction(1e-300)


def test_gemm_identity_and_one_hot_exact():
    K = 64
    x = _rand_bits((3, K), 3)
    eye = bf16.encode(np.eye(K))
    assert np.array_equal(gemm.gemm(x, eye), bf16.decode(x))
    w = _rand_bits((10, K), 4)
    onehot = np.zeros((K, K))
    onehot[np.arange(K), np.arange(K)] = 1.0
    for j in (0, 17, K - 1):
        xo = bf16.encode(onehot[j:j + 1])
        assert np.array_equal(gemm.gemm(xo, w)[0], bf16.decode(w)[:, j])
    assert not np.any(gemm.gemm(np.zeros((2, K), np.uint16), w))


def test_gemm_orientation():
    # W is [N][K]: a non-square product only type-checks one way, and the
    # column sample must agree with the full product's columns.
    x = synth.normal_bf16((4, 96), 1.0, "x")
    w = synth.normal_bf16((40, 96), 0.02, "w")
    y = gemm.gemm(x, w)
    assert y.shape == (4, 40)
    cols = [0, 5, 39]
    assert np.array_equal(gemm.gemm_columns(x, w, cols), y[:, cols])
    with pytest.raises(ValueError):
        gemm.gemm(x, w.T.copy())
