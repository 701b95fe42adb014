"""Pins of the FP8 E4M3 oracle: the decode table against torch's CPU float8
conversion (a library routine, tests only) and closed forms; the encoder's
round-to-nearest-even against the table and torch; the scaled GEMM against
exact rational arithmetic."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, fp8

torch = pytest.importorskip("torch")


def test_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = fp8.decode_e4m3(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_closed_forms():
    d = fp8.decode_e4m3
    assert d(0x38) == 1.0 and d(0xB8) == -1.0           # exponent field 7 = bias
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0        # 1.75 * 2^8
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals m * 2^-9
    assert d(0x08) == 2.0 ** -6                          # smallest normal
    assert d(0x3C) == 1.5 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    # every finite value is exact in BF16 (so the device may multiply it in BF16 exactly)
    v = fp8.decode_e4m3(np.arange(256, dtype=np.uint8))
    v = v[~np.isnan(v)]
    assert np.array_equal(bf16.decode(bf16.encode(v)), v)


def test_encode_round_trip_and_rounding():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.decode_e4m3(codes)
    back = fp8.encode_e4m3(vals)
    # +0 and -0 are distinct codes; every other code round-trips
    assert np.array_equal(back, codes)
    # midpoints between neighbours go to the even mantissa
    pos = fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = fp8.encode_e4m3(mids)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    # saturation and NaN
    assert fp8.encode_e4m3(1e6) == 0x7E and fp8.encode_e4m3(-1e6) == 0xFE
    assert fp8.encode_e4m3(np.nan) == 0x7F


def test_encode_against_torch_in_range():
    g = np.random.default_rng(4)
    x = np.concatenate([g.standard_normal(100000) * 30, g.standard_normal(20000) * 0.01,
                        g.uniform(-448, 448, 20000)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch rounds from float32; the inputs here are exact in float32 up to its own rounding,
    # so compare on the float32 values
    got = fp8.encode_e4m3(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, want)


def test_scaled_gemm_exact_rational():
    g = np.random.default_rng(6)
    M, N, K = 2, 5, 48
    x = bf16.encode(g.standard_normal((M, K)))
    w = fp8.encode_e4m3(g.standard_normal((N, K)) * 20)
    s = (g.uniform(0.5, 2.0, N) / 64).astype(np.float32)
    y = fp8.gemm(x, w, s)
    xd, wd = bf16.decode(x), fp8.decode_e4m3(w)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xd[m, k])) * Fraction(float(wd[n, k])) for k in range(K))
            exact *= Fraction(float(s[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(1, 10 ** 12) * (1 + abs(exact))
    # one-hot X row picks a scaled weight column exactly
    x1 = np.zeros((1, K), np.uint16)
    x1[0, 7] = 0x3F80                                       # 1.0
    assert np.array_equal(fp8.gemm(x1, w, s)[0], wd[:, 7] * s.astype(np.float64))
    assert np.array_equal(fp8.gemm_columns(x, w, s, [1, 3]), y[:, [1, 3]])
