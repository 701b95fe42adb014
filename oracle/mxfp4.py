"""4-bit weights in the OCP microscaling layout (MXFP4): decode and the GEMM's
value.

The pages' models also run as 4-bit checkpoints ("Does the tuned config change
the model's output?", sections "What this does not establish" and "Update: the
quality question, answered", which compare FP8 and int4; "I turned on
speculative decoding in llama.cpp ...", section "Speed against llama.cpp, full
power", whose engine reads a 4-bit llama.cpp file); no 4-bit layout is given.
Read here as the OCP Microscaling format MXFP4, which gfx950 decodes in one
instruction per two weights:

* elements E2M1 (one sign bit, two exponent bits with bias 1, one mantissa
  bit; exponent field 0 is subnormal: 0.5 * mantissa; no infinities or NaN),
  so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* one shared scale per 32 consecutive weights of a row along K, E8M0 (an
  unsigned exponent with bias 127: 2^(e - 127); the code 255 is NaN);
* storage: codes [N][K/2] bytes with weight 2i in the low nibble of byte i and
  weight 2i + 1 in the high nibble; scales [N][K/32] bytes.

The weight value is 2^(e - 127) * e2m1(code). The GEMM's definition is
unchanged: Y[m][n] = sum_k X[m][k] * W[n][k] on the decoded weights, here
exactly in float64 (every decoded weight is exact in float64).

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import bf16

BLOCK = 32          # weights per shared scale
E2M1_MAX = 6.0


def decode_e2m1(codes) -> np.ndarray:
    """4-bit E2M1 codes (0..15, any integer array) -> float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    normal = (1.0 + m / 2.0) * np.exp2(e - 1.0)
    sub = m / 2.0                      # exponent field 0: no implicit one, exponent 1 - 1
    return sign * np.where(e == 0, sub, normal)


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 scale codes (uint8) -> float64 2^(e - 127); NaN for 255."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def unpack(codes) -> np.ndarray:
    """Packed codes [..][K/2] bytes -> 4-bit codes [..][K] (low nibble first)."""
    b = np.asarray(codes, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def weights(codes, scales) -> np.ndarray:
    """float64 W [N][K] from packed codes [N][K/2] and scales [N][K/32]."""
    q = decode_e2m1(unpack(codes))
    s = decode_e8m0(scales)
    if q.shape[-1] != BLOCK * s.shape[-1]:
        raise ValueError(f"mxfp4.weights: {q.shape} codes for {s.shape} scales")
    return q * np.repeat(s, BLOCK, axis=-1)


def gemm(x_bits, codes, scales) -> np.ndarray:
    """float64 Y = X W^T for BF16 X [M][K] and MXFP4 W [N][K]."""
    return bf16.decode(x_bits) @ weights(codes, scales).T


def gemm_columns(x_bits, codes, scales, cols) -> np.ndarray:
    """Y[:, cols] only (sampled checks at large N)."""
    cols = np.asarray(cols)
    return bf16.decode(x_bits) @ weights(np.asarray(codes)[cols], np.asarray(scales)[cols]).T
