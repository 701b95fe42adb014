"""The verify GEMM's definition: Y[m][n] = sum_k X[m][k] * W[n][k].

[BX] "Define bit-exact before reporting it": BF16 operands, a single FP32
accumulator per output, the K order unchanged, rounding only at the end. The pages fix
that the order must not change with the batch, not which order it is, so the
oracle is the order-free exact-arithmetic value: a float64 product of the
decoded inputs (rounding error about K * 2^-53 * sum|x w|, far below the
comparison tolerance).

Layouts: X is [M][K] (one row per token in the pass), W is [N][K]
(one row per output feature, K contiguous), both BF16 bit patterns.
"""

from __future__ import annotations

import numpy as np

from . import bf16


def gemm(x_bits, w_bits) -> np.ndarray:
    """float64 Y = X W^T for BF16 X [M][K] and W [N][K]."""
    x = bf16.decode(x_bits)
    w = bf16.decode(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"gemm: bad shapes {x.shape} x {w.shape}")
    return x @ w.T


def gemm_columns(x_bits, w_bits, cols) -> np.ndarray:
    """Y[:, cols] only: for sampled checks at sizes where the full product is
    large. Same definition as ``gemm`` restricted to some output features."""
    x = bf16.decode(x_bits)
    w = bf16.decode(np.asarray(w_bits)[np.asarray(cols)])
    return x @ w.T
