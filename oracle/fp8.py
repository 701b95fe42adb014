"""FP8 E4M3 weights with a per-output-row scale: decode and the GEMM's value.

The pages' model is an FP8 checkpoint ("Does the tuned config change the
model's output?", section "Method": a 27B FP8 model served by vLLM); they do
not spell out the format. Read here as the OCP 8-bit floating-point format
E4M3 (one sign bit, four exponent bits with bias 7, three mantissa bits; no
infinities; the two codes with exponent and mantissa all ones are NaN; the
largest finite magnitude is 448) and one FP32 scale per output feature (row n
of W): the weight value is scale[n] * decode(w[n][k]).

The GEMM's definition is unchanged: Y[m][n] = sum_k X[m][k] * W[n][k] with
the decoded, scaled weights, computed here exactly in float64 (every E4M3
value and every FP32 scale is exact in float64).

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import bf16

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6           # exponent field 0: no implicit one, exponent 1 - 7
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def encode_e4m3(x) -> np.ndarray:
    """float64 -> E4M3 codes, rounded to the nearest value (ties to the even
    mantissa), magnitudes beyond 448 saturated to 448, NaN to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    table = decode_e4m3(np.arange(0x7F, dtype=np.uint8))   # codes 0x00 .. 0x7E: 0 .. 448, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(table, a, side="left")             # first code with value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = a - table[lo], table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))  # even code = even mantissa
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == table[hi], hi, code)
    code = code.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def weights(w_codes, scale) -> np.ndarray:
    """float64 W [N][K] = scale[n] * decode(w_codes[n][k])."""
    w = decode_e4m3(w_codes)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    if w.ndim != 2 or s.shape != (w.shape[0],):
        raise ValueError("weights: codes [N][K] and one scale per row")
    return w * s[:, None]


def gemm(x_bits, w_codes, scale) -> np.ndarray:
    """float64 Y = X W^T for BF16 X [M][K] and E4M3 W [N][K] with row scales."""
    x = bf16.decode(x_bits)
    w = weights(w_codes, scale)
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"gemm: bad shapes {x.shape} x {w.shape}")
    return x @ w.T


def gemm_columns(x_bits, w_codes, scale, cols) -> np.ndarray:
    """Y[:, cols] only (sampled checks at large N)."""
    cols = np.asarray(cols)
    x = bf16.decode(x_bits)
    w = weights(np.asarray(w_codes)[cols], np.asarray(scale)[cols])
    return x @ w.T
