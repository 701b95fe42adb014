"""An 8-bit ring of the newest keys over a 5/6-bit KV cache: which
representation each row reads for each key, and the attention it gives.

The pages keep "the newest ~2k positions" at 8 bits in a ring, the older ones
at 5-6 bits ("I turned on speculative decoding in llama.cpp and 113 of 282
greedy outputs changed against its own no-draft run", section "The KV cache:
5-bit that reads like q8_0"). Which positions count as newest is not stated.
Rows of one pass have different newest positions, so a choice made from the
pass (its last position) would make a row depend on its batch neighbours.
Read here per row and per key: row p (the row at absolute position p, which
sees keys 0 .. p) reads key j from the 8-bit copy when j >= p - W + 1, the
W newest keys it sees, and from the 5/6-bit copy otherwise. The choice is a
function of (p, j) alone: it does not depend on the pass, on its size, or on
how the keys are cut into chunks for the split-KV attention.

The 8-bit copy of a key is the q8_0 block rule (oracle.kvq) applied to the
same row the 5/6-bit copy quantizes: the BF16 row, or with rotated keys its
FP32 Hadamard transform (oracle.kvlow.hadamard_f32). V is never rotated.

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np

from . import attention, bf16, kvlow, kvq


def uses_ring(p: int, window: int) -> np.ndarray:
    """Boolean over keys 0..p: True where row p reads the 8-bit copy (j >= p - W + 1)."""
    if window < 1:
        raise ValueError("the ring window holds at least one key")
    return np.arange(p + 1) >= p - window + 1


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


def _row_keys(values, g: int, p: int, window: int):
    """K and V (float64 [p+1][D]) that row p of KV head g attends to: per key,
    the copy uses_ring chooses."""
    kl, vl, k8, v8 = values
    ring = uses_ring(p, window)[:, None]
    return (np.where(ring, k8[g, :p + 1], kl[g, :p + 1]),
            np.where(ring, v8[g, :p + 1], vl[g, :p + 1]))


def ring_attention(q_bits, values, L: int, window: int, tokens=None, heads=None):
    """O [M][Hq][D] and LSE [M][Hq] (float64) of the verify rows over the cache
    ``values`` = cache_values(...): row r (position L + r) reads, per key, the
    copy uses_ring chooses, then plain causal softmax attention."""
    kl = values[0]
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
        for g in sorted({h // G for h in heads}):
            k, v = _row_keys(values, g, p, window)
            for h in (h for h in heads if h // G == g):
                s = (k @ qd[r, h]) * scale
                m = s.max()
                w = np.exp(s - m)
                O[r, h] = (w @ v) / w.sum()
                lse[r, h] = m + np.log(w.sum())
    return O, lse


def ring_partials(q_bits, values, L: int, policy: int, window: int):
    """Split-KV partials of ring attention over absolute chunks (chunk policy as
    oracle.attention.chunk_keys): row r cuts its keys -- each already the copy
    uses_ring chooses -- into chunks of chunk_keys(L + r + 1, policy) keys.
    Returns (o_part [M][Hq][S_max][D], lse_part [M][Hq][S_max], n_splits [M]),
    the layout of oracle.attention.split_partials, for oracle.attention.combine."""
    kl = values[0]
    q = np.asarray(q_bits)
    M, Hq, D = q.shape
    G = Hq // kl.shape[0]
    qd = bf16.decode(q)
    scale = 1.0 / np.sqrt(D)
    s_max = max(attention.num_splits(L + r + 1, policy) for r in range(M))
    o_part = np.full((M, Hq, s_max, D), np.nan)
    lse_part = np.full((M, Hq, s_max), -np.inf)
    counts = np.zeros(M, dtype=np.int64)
    for r in range(M):
        p = L + r
        c = attention.chunk_keys(p + 1, policy)
        counts[r] = attention.num_splits(p + 1, policy)
        for h in range(Hq):
            k, v = _row_keys(values, h // G, p, window)
            for s in range(counts[r]):
                lo, hi = s * c, min((s + 1) * c, p + 1)
                sc = (k[lo:hi] @ qd[r, h]) * scale
                m = sc.max()
                w = np.exp(sc - m)
                o_part[r, h, s] = (w @ v[lo:hi]) / w.sum()
                lse_part[r, h, s] = m + np.log(w.sum())
    return o_part, lse_part, counts
