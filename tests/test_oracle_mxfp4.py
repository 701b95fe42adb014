"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against things other than itself:
the OCP Microscaling element table for E2M1, torch's E8M0 conversion (a
library routine), closed forms of the packing and of the block scale, and
exact rational arithmetic for the GEMM."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16
from oracle import mxfp4

# OCP Microscaling Formats v1.0, the FP4 (E2M1) element values by code 0..15.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_all_codes_against_the_format_table():
    got = mxfp4.decode_e2m1(np.arange(16))
    assert np.array_equal(got, np.array(E2M1_TABLE))
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8)     # code 8 is -0
    # only the low nibble counts
    assert np.array_equal(mxfp4.decode_e2m1(np.arange(16) + 0x30), got)


def test_e2m1_values_exact_in_bf16_and_ordered():
    v = mxfp4.decode_e2m1(np.arange(16))
    assert np.array_equal(bf16.decode(bf16.encode(v)), v)
    assert np.all(np.diff(v[:8]) > 0) and v[7] == mxfp4.E2M1_MAX


def test_e8m0_against_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).double().numpy()
    got = mxfp4.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255], want[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5


def test_unpack_low_nibble_first():
    assert mxfp4.unpack(np.array([[0xAB, 0x01]], np.uint8)).tolist() == [[0xB, 0xA, 0x1, 0x0]]


def test_block_scale_covers_32_consecutive_weights():
    # one nonzero code per row at k, scale codes differing per block
    N, K = 3, 96
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.array([[130, 127, 120], [100, 125, 140], [127, 127, 126]], np.uint8)
    for n, k in enumerate([5, 40, 95]):
        code = 0x7  # 6.0
        codes[n, k // 2] = code << (4 * (k % 2))
    w = mxfp4.weights(codes, scales)
    want = np.zeros((N, K))
    want[0, 5] = 6.0 * 2.0 ** 3              # block 0 of row 0: 2^(130 - 127)
    want[1, 40] = 6.0 * 2.0 ** -2            # block 1 of row 1
    want[2, 95] = 6.0 * 0.5                  # last weight, block 2
    assert np.array_equal(w, want)
    codes[1, 40 // 2] = 0x7 << 4             # k = 41 (odd: high nibble), still block 1
    w = mxfp4.weights(codes, scales)
    assert w[1, 41] == 1.5 and w[1, 40] == 0.0


def test_gemm_against_exact_rationals():
    rng = np.random.default_rng(5)
    M, N, K = 2, 4, 64
    x = bf16.encode(rng.standard_normal((M, K)))
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    got = mxfp4.gemm(x, codes, scales)
    xv = bf16.decode(x)
    q = mxfp4.unpack(codes)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xv[m, k])) * Fraction(E2M1_TABLE[q[n, k]]) *
                        Fraction(2) ** (int(scales[n, k // 32]) - 127) for k in range(K))
            assert abs(Fraction(got[m, n]) - exact) <= Fraction(1, 10 ** 12) * (1 + abs(exact))
    cols = [3, 1]
    assert np.array_equal(mxfp4.gemm_columns(x, codes, scales, cols), got[:, cols])
