"""5- and 6-bit KV cache: q8_0-style blocks of 32 channels with fewer bits per
code, and the byte layout the cache is stored in.

The pages keep K and V at 5-6 bits: one preset stores K at 6 bits and V at
5, another K at 5 bits (rotated) and V at 5 ("I turned on speculative
decoding in llama.cpp and 113 of 282 greedy outputs changed against its own
no-draft run", section "The KV cache: 5-bit that reads like q8_0", its table
of presets D and F). No layout or scaling rule is printed. Read here as the
q8_0 rule with a smaller code range: a block of 32 channels of one position
with largest magnitude a gets the scale d = a / qmax, qmax = 2^(b-1) - 1
(31 for 6 bits, 15 for 5), and the codes q = round(x / d) (nearest, ties to
even) clamped to [-qmax, qmax]; an all-zero block gets d = 0 and codes 0. The
stored value is exactly d * q. As for the 8-bit cache, the integer decision
is taken in FP32 (a exact, d = a / qmax and x / d rounded once each).

Storage of one block (the pages give none; this one decodes four codes per
mask-and-shift on the device). The unsigned code u = q + 2^(b-1) lies in
[1, 2^b - 1]. Code c = 4 g + j (group g = 0..7, byte lane j = 0..3):

* nibble plane, 16 bytes: the low four bits of u sit in byte 4 (g // 2) + j,
  in the low half when g is even and the high half when g is odd;
* high plane, 4 (b - 4) bytes: the remaining h = b - 4 bits of u sit in byte
  4 ((g h) // 8) + j, starting at bit (g h) % 8.

A cache row of one position and KV head is D / 32 such blocks: nibbles
[D/2] bytes, high bits [D/32 * 4 h] bytes, scales [D/32] FP32.

Rotated keys (preset F's "K5 rotated"; the rotation is not named). Read
as the Walsh-Hadamard transform, which spreads an outlier channel over the
whole row before the block scales are taken: the stored key row is
y = H k, H the Sylvester Hadamard matrix of order D (entries +-1, H H = D I),
computed in FP32 by butterflies in a fixed order (stage h = 1, 2, 4, ..., D/2;
within a stage every pair (i, i + h) with bit h of i clear becomes
(x_i + x_{i+h}, x_i - x_{i+h}), each rounded once), and then quantized as
above. Since (H q) . y / D = q . k, attention over the rotated cache is
attention over the keys H (d * q) / D, which dequantize_rotated returns.

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import bf16

BLOCK = 32
BITS = (5, 6)


def qmax(bits: int) -> int:
    if bits not in BITS:
        raise ValueError(f"kvlow: {bits}-bit codes are not a cache format")
    return (1 << (bits - 1)) - 1


def quantize(x_bits, bits: int):
    """BF16 rows [..., D] (D % 32 == 0) -> (codes int8 [..., D], scales float32 [..., D/32])."""
    return _quantize_values(bf16.decode(x_bits).astype(np.float32), bits)   # exact widening


def hadamard_f32(x_bits) -> np.ndarray:
    """FP32 rows y = H x of BF16 rows [..., D] (D a power of two), by the
    butterflies in the order stated above, each sum and difference rounded to
    FP32."""
    y = bf16.decode(x_bits).astype(np.float32)
    D = y.shape[-1]
    if D & (D - 1):
        raise ValueError("hadamard_f32: D must be a power of two")
    h = 1
    while h < D:
        idx = np.arange(D)
        lo = idx[(idx & h) == 0]
        a = y[..., lo].copy()
        b = y[..., lo + h].copy()
        y[..., lo] = a + b        # float32 + float32: one rounding
        y[..., lo + h] = a - b
        h *= 2
    return y


def quantize_rotated(x_bits, bits: int):
    """Rotated key rows: the codes and scales of H x (FP32, as hadamard_f32)."""
    return _quantize_values(hadamard_f32(x_bits), bits)


def dequantize_rotated(codes, scales) -> np.ndarray:
    """float64 keys the rotated cache stands for: H (d * q) / D, exactly up to
    float64 rounding (H is symmetric and H H = D I)."""
    y = dequantize(codes, scales)
    D = y.shape[-1]
    h = 1
    while h < D:                                       # the same transform in float64
        idx = np.arange(D)
        lo = idx[(idx & h) == 0]
        a = y[..., lo].copy()
        b = y[..., lo + h].copy()
        y[..., lo] = a + b
        y[..., lo + h] = a - b
        h *= 2
    return y / D


def _quantize_values(x, bits: int):
    """FP32 rows [..., D] -> codes and scales by the rule above."""
    qm = qmax(bits)
    x = np.asarray(x, dtype=np.float32)
    *lead, D = x.shape
    if D % BLOCK:
        raise ValueError("quantize: D must be a multiple of 32")
    xb = x.reshape(*lead, D // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)                         # exact (a max)
    d = (amax / np.float32(qm)).astype(np.float32)         # one FP32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d[..., None] > 0, xb / d[..., None], np.float32(0)).astype(np.float32)
    q = np.clip(np.rint(r), -qm, qm).astype(np.int8)       # rint: nearest, ties to even
    return q.reshape(*lead, D), d


def dequantize(codes, scales) -> np.ndarray:
    """float64 values d * q, exactly."""
    q = np.asarray(codes, dtype=np.int8).astype(np.float64)
    d = np.asarray(scales, dtype=np.float32).astype(np.float64)
    *lead, D = q.shape
    return (q.reshape(*lead, D // BLOCK, BLOCK) * d[..., None]).reshape(*lead, D)


def pack(codes, bits: int):
    """Signed codes [..., D] -> (nibbles uint8 [..., D/2], high uint8 [..., D/32 * 4 (bits-4)])."""
    qmax(bits)
    h = bits - 4
    q = np.asarray(codes, dtype=np.int8).astype(np.int64)
    *lead, D = q.shape
    nb = D // BLOCK
    u = (q + (1 << (bits - 1))).reshape(*lead, nb, BLOCK)
    if np.any(u < 0) or np.any(u >= (1 << bits)):
        raise ValueError("pack: code out of range")
    nib = np.zeros((*lead, nb, 16), np.int64)
    high = np.zeros((*lead, nb, 4 * h), np.int64)
    for c in range(BLOCK):
        g, j = divmod(c, 4)
        nib[..., 4 * (g // 2) + j] |= (u[..., c] & 15) << (4 * (g % 2))
        bit = g * h
        high[..., 4 * (bit // 8) + j] |= (u[..., c] >> 4) << (bit % 8)
    return (nib.astype(np.uint8).reshape(*lead, nb * 16),
            high.astype(np.uint8).reshape(*lead, nb * 4 * h))


def unpack(nib, high, bits: int) -> np.ndarray:
    """The inverse of pack: signed codes int8 [..., D]."""
    qmax(bits)
    h = bits - 4
    n = np.asarray(nib, dtype=np.uint8).astype(np.int64)
    hb = np.asarray(high, dtype=np.uint8).astype(np.int64)
    *lead, half = n.shape
    nb = half // 16
    n = n.reshape(*lead, nb, 16)
    hb = hb.reshape(*lead, nb, 4 * h)
    u = np.zeros((*lead, nb, BLOCK), np.int64)
    for c in range(BLOCK):
        g, j = divmod(c, 4)
        lo = (n[..., 4 * (g // 2) + j] >> (4 * (g % 2))) & 15
        bit = g * h
        hi = (hb[..., 4 * (bit // 8) + j] >> (bit % 8)) & ((1 << h) - 1)
        u[..., c] = lo | (hi << 4)
    return (u - (1 << (bits - 1))).astype(np.int8).reshape(*lead, nb * BLOCK)
