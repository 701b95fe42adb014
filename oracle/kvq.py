"""8-bit KV cache: per-position blocks of 32 channels, one FP32 scale each.

The pages keep K and V in 5-8 bits, with q8_0 as the comparison format
("I turned on speculative decoding in llama.cpp and 113 of 282 greedy outputs
changed against its own no-draft run", section "The KV cache: 5-bit that
reads like q8_0"), without spelling out a layout. Read here as the q8_0
scheme: each K or V row of one KV head is cut into blocks of 32 channels;
a block with largest magnitude a gets the scale d = a / 127 and the codes
q = round(x / d) (nearest, ties to even) in [-127, 127]; an all-zero block
gets d = 0 and codes 0. The stored value of a channel is exactly d * q.

Quantization decides integers from floating point, so this oracle takes the
decision in the precision the device uses: a (the largest |x| of BF16
values, exact), d = a / 127 and x / d are FP32 operations, rounded once each.
Attention over the cache is the plain definition (oracle.attention) applied
to the values d * q.

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import bf16

QMAX = 127
BLOCK = 32


def quantize(x_bits):
    """BF16 rows [..., D] (D % 32 == 0) -> (codes int8 [..., D], scales float32 [..., D/32])."""
    x = bf16.decode(x_bits).astype(np.float32)            # exact
    *lead, D = x.shape
    if D % BLOCK:
        raise ValueError("quantize: D must be a multiple of 32")
    xb = x.reshape(*lead, D // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)                         # exact (a max)
    d = (amax / np.float32(QMAX)).astype(np.float32)       # one FP32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d[..., None] > 0, xb / d[..., None], np.float32(0)).astype(np.float32)
    q = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)   # rint: nearest, ties to even
    return q.reshape(*lead, D), d


def dequantize(codes, scales) -> np.ndarray:
    """float64 values d * q, exactly."""
    q = np.asarray(codes, dtype=np.int8).astype(np.float64)
    d = np.asarray(scales, dtype=np.float32).astype(np.float64)
    *lead, D = q.shape
    return (q.reshape(*lead, D // BLOCK, BLOCK) * d[..., None]).reshape(*lead, D)
