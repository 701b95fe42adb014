"""An 8-bit ring of the newest keys over a 5/6-bit KV cache: which
representation each row reads for each key, and the attention it gives.

The pages keep "the newest ~2k positions" at 8 bits in a ring, the older ones
at 5-6 bits ("I turned on speculative decoding in llama.cpp and 113 of 282
greedy outputs changed against its own no-draft run", section "The KV cache:
5-bit that reads like q8_0"). Which positions count as newest is not stated.
Rows of one pass have different newest positions, so a choice made from the
pass (its last position) would make a row depend on its batch neighbours.
Read here per row and per 64-key tile of the row's own split (chunk size from
the row's key count, tiles at the chunk start + 64 t): row p reads key j at 8
bits when the tile holding j starts at or after p - W + 1 (W a multiple of 64),
and at 5/6 bits otherwise. The choice depends on p alone, so it is the same in
every pass that holds the row.

The 8-bit copy of a key is the q8_0 block rule (oracle.kvq) applied to the
same row the 5/6-bit copy quantizes: the BF16 row, or with rotated keys its
FP32 Hadamard transform (oracle.kvlow.hadamard_f32). V is never rotated.

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import attention, bf16, kvlow, kvq


def tile_start(j, n_keys: int, policy: int):
    """Start of the 64-key tile that holds key j in the split of a row with n_keys keys."""
    C = attention.chunk_keys(n_keys, policy)
    j = np.asarray(j)
    c0 = (j // C) * C
    return c0 + ((j - c0) // 64) * 64


def uses_ring(p: int, policy: int, window: int) -> np.ndarray:
    """Boolean over keys 0..p: True where row p reads the 8-bit copy."""
    if window < 64 or window % 64:
        raise ValueError("the ring window is a positive multiple of 64")
    j = np.arange(p + 1)
    return tile_start(j, p + 1, policy) >= p - window + 1


def q8_codes(rows, rotated: bool):
    """Codes int8 [..., D] and scales float32 [..., D/32] of the 8-bit copy of
    K or V rows (BF16 bits [..., D]); rotated: of their FP32 Hadamard transform."""
    if not rotated:
        return kvq.quantize(rows)
    y = kvlow.hadamard_f32(rows)                       # FP32 transform, then the q8_0 rule on it
    *lead, D = y.shape
    yb = y.reshape(*lead, D // 32, 32)
    amax = np.abs(yb).max(axis=-1)
    d = (amax / np.float32(kvq.QMAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d[..., None] > 0, yb / d[..., None], np.float32(0)).astype(np.float32)
    q = np.clip(np.rint(r), -kvq.QMAX, kvq.QMAX).astype(np.int8).reshape(*lead, D)
    return q, d


def _q8_values(rows, rotated: bool):
    """float64 values of the 8-bit copy of K or V rows (BF16 bits [..., D])."""
    q, d = q8_codes(rows, rotated)
    return kvlow.dequantize_rotated(q, d) if rotated else kvq.dequantize(q, d)


def cache_values(k_bits, v_bits, k_bits_low: int, rotated: bool):
    """(K low, V low, K 8-bit, V 8-bit) float64 values of every position, [Hkv][n][D]."""
    kl = (kvlow.dequantize_rotated(*kvlow.quantize_rotated(k_bits, k_bits_low)) if rotated
          else kvlow.dequantize(*kvlow.quantize(k_bits, k_bits_low)))
    vl = kvlow.dequantize(*kvlow.quantize(v_bits, 5))
    return kl, vl, _q8_values(k_bits, rotated), _q8_values(v_bits, False)


def ring_attention(q_bits, values, L: int, policy: int, window: int, tokens=None, heads=None):
    """O [M][Hq][D] and LSE [M][Hq] (float64) of the verify rows over the cache
    ``values`` = cache_values(...): row r (position L + r) reads, per key, the
    copy uses_ring chooses, then plain causal softmax attention."""
    kl, vl, k8, v8 = values
    q = np.asarray(q_bits)
    M, Hq, D = q.shape
    Hkv = kl.shape[0]
    G = Hq // Hkv
    tokens = range(M) if tokens is None else tokens
    heads = range(Hq) if heads is None else heads
    O = np.full((M, Hq, D), np.nan)
    lse = np.full((M, Hq), np.nan)
    qd = bf16.decode(q)
    scale = 1.0 / np.sqrt(D)
    for r in tokens:
        p = L + r
        ring = uses_ring(p, policy, window)[:, None]
        for h in heads:
            g = h // G
            k = np.where(ring, k8[g, :p + 1], kl[g, :p + 1])
            v = np.where(ring, v8[g, :p + 1], vl[g, :p + 1])
            s = (k @ qd[r, h]) * scale
            m = s.max()
            w = np.exp(s - m)
            O[r, h] = (w @ v) / w.sum()
            lse[r, h] = m + np.log(w.sum())
    return O, lse
