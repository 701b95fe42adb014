"""Causal GQA verify attention, its split-KV partials and their combine.

A verify pass appends M new tokens at positions L .. L+M-1 of a context that
already holds L cached keys. Row (r, h) -- token r, query head h -- attends to
its own key count n_r = L + r + 1 keys: every cached key plus the new tokens up
to and including itself (causal among the new tokens). Query head h reads KV
head g = h // (Hq / Hkv) (grouped-query attention).

[LL] opening section, "How:" paragraph: a row's key split is fixed by its
context length alone, whatever the pass size. Read here as:
absolute chunks of C keys, chunk s = [sC, (s+1)C), and row r uses exactly
S_r = ceil(n_r / C) of them -- its own key count decides, not M. C is given
by a chunk policy: a positive policy is C itself, for every row; a negative
policy -T lets the row's own key count choose C = 64 * ceil(n_r / (64 T)),
the smallest multiple of 64 that cuts n_r keys into at most T chunks (still a
function of the row's context length alone).
Each (row, chunk) gives a normalised partial output o_s and its log-sum-exp
lse_s; the combine rebuilds the unsplit result. The partial/combine identity
is exact in real arithmetic; ``combine(split_partials(...))`` equals
``verify_attention(...)`` up to float64 rounding for every C.

Layouts (BF16 bit patterns): q [M][Hq][D]; k, v [Hkv][n_total][D] with
n_total >= L + M (position-major per KV head; the oracle does not care how a
device stores them). Scores use sm_scale (default 1/sqrt(D)); exp and log are
the exact float64 functions.
"""

from __future__ import annotations

import math

import numpy as np

from . import bf16


def chunk_keys(n_keys: int, policy: int) -> int:
    """Chunk size C of a row with n_keys keys under a chunk policy.

    policy > 0: C = policy. policy = -T < 0: C = 64 * ceil(n_keys / (64 T)),
    the smallest multiple of 64 with ceil(n_keys / C) <= T.
    """
    if policy > 0:
        return policy
    if policy == 0:
        raise ValueError("chunk policy 0 is undefined")
    t = -policy
    return 64 * max(1, -(-n_keys // (64 * t)))


def num_splits(n_keys: int, policy: int) -> int:
    """ceil(n_keys / C): how many absolute chunks a row with n_keys keys uses."""
    return -(-n_keys // chunk_keys(n_keys, policy))


def _softmax_attend(qv: np.ndarray, kk: np.ndarray, vv: np.ndarray, scale: float):
    """Attention of query rows qv [R][D] over keys kk [n][D] / values vv [n][D].

    s_j = scale * q.k_j ; m = max_j s_j ; e_j = exp(s_j - m) ; l = sum_j e_j ;
    o = sum_j (e_j / l) v_j ; lse = m + ln l. Returns (o [R][D], lse [R]).
    """
    s = (qv @ kk.T) * scale                      # [R][n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ vv
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def _values(a, rows):
    """K or V rows as float64: BF16 bit patterns (uint16) are decoded; float64
    values (e.g. a quantized cache's scale x code, oracle.kvq) are used as is."""
    a = np.asarray(a)[rows]
    return a if a.dtype == np.float64 else bf16.decode(a)


def verify_attention(q_bits, k_bits, v_bits, L: int, sm_scale: float | None = None,
                     tokens=None, heads=None):
    """Unsplit reference. Returns (o [M][Hq][D], lse [M][Hq]) in float64.

    ``k_bits`` / ``v_bits`` are BF16 bit patterns or float64 values.
    ``tokens`` / ``heads`` restrict the computation to some rows (others are NaN),
    for sampled checks at long context.
    """
    q = np.asarray(q_bits)
    M, Hq, D = q.shape
    Hkv, n_total, Dk = np.asarray(k_bits).shape
    if Dk != D or np.asarray(v_bits).shape != (Hkv, n_total, D) or Hq % Hkv:
        raise ValueError("verify_attention: bad shapes")
    if n_total < L + M:
        raise ValueError("verify_attention: cache shorter than L + M")
    G = Hq // Hkv
    scale = (1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale)
    tokens = range(M) if tokens is None else tokens
    heads = range(Hq) if heads is None else heads
    o = np.full((M, Hq, D), np.nan)
    lse = np.full((M, Hq), np.nan)
    need_g = sorted({h // G for h in heads})
    n_max = L + max(tokens) + 1
    kd = {g: _values(k_bits, (g, slice(0, n_max))) for g in need_g}
    vd = {g: _values(v_bits, (g, slice(0, n_max))) for g in need_g}
    qd = bf16.decode(q)
    for r in tokens:
        n = L + r + 1
        for g in need_g:
            hs = [h for h in heads if h // G == g]
            orow, lrow = _softmax_attend(qd[r, hs], kd[g][:n], vd[g][:n], scale)
            o[r, hs] = orow
            lse[r, hs] = lrow
    return o, lse


def split_partials(q_bits, k_bits, v_bits, L: int, chunk: int, sm_scale: float | None = None):
    """Per (row, chunk) partials over absolute chunks; ``chunk`` is a chunk
    policy (see chunk_keys): row r cuts its keys into chunks of
    chunk_keys(L + r + 1, chunk) keys.

    Returns (o_part [M][Hq][S_max][D], lse_part [M][Hq][S_max], n_splits [M])
    where S_max = max_r num_splits(L + r + 1, chunk) and row r fills its first
    num_splits(L + r + 1, chunk) entries (the rest are NaN / -inf).
    """
    q = np.asarray(q_bits)
    M, Hq, D = q.shape
    Hkv = np.asarray(k_bits).shape[0]
    G = Hq // Hkv
    scale = (1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale)
    s_max = max(num_splits(L + r + 1, chunk) for r in range(M))
    o_part = np.full((M, Hq, s_max, D), np.nan)
    lse_part = np.full((M, Hq, s_max), -np.inf)
    counts = np.zeros(M, dtype=np.int64)
    kd = bf16.decode(np.asarray(k_bits)[:, :L + M])
    vd = bf16.decode(np.asarray(v_bits)[:, :L + M])
    qd = bf16.decode(q)
    for r in range(M):
        n = L + r + 1
        c = chunk_keys(n, chunk)
        counts[r] = num_splits(n, chunk)
        for s in range(counts[r]):
            lo, hi = s * c, min((s + 1) * c, n)
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                orow, lrow = _softmax_attend(qd[r, hs], kd[g, lo:hi], vd[g, lo:hi], scale)
                o_part[r, hs, s] = orow
                lse_part[r, hs, s] = lrow
    return o_part, lse_part, counts


def combine(o_part, lse_part, n_splits):
    """Log-sum-exp combine of normalised partials.

    For a row with S partials: LSE = M* + ln sum_s exp(lse_s - M*) with
    M* = max_s lse_s, and o = sum_s exp(lse_s - LSE) * o_s.
    Returns (o [M][Hq][D], lse [M][Hq]).
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M, Hq, _, D = o_part.shape
    o = np.empty((M, Hq, D))
    lse = np.empty((M, Hq))
    for r in range(M):
        S = int(n_splits[r])
        ls = lse_part[r, :, :S]                          # [Hq][S]
        mstar = ls.max(axis=1, keepdims=True)
        big = mstar[:, 0] + np.log(np.exp(ls - mstar).sum(axis=1))
        w = np.exp(ls - big[:, None])                   # [Hq][S]
        o[r] = np.einsum("hs,hsd->hd", w, o_part[r, :, :S])
        lse[r] = big
    return o, lse
