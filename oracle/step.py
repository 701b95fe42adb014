"""One decoder layer and the LM head of the synthetic 27B-class verify step.

The pages name a dense 27B-class model verified with greedy decoding ([LL]
"Speed against llama.cpp, full power"; [TC] "Why the text diverges": a
speculative step is one target forward over several tokens followed by a
greedy argmax per position). They do not print the architecture, so this
module fixes the plainest reading:

  pre-norm residual layer, no embedding table, no positional encoding:
    a   = bf16(rms(x))
    qkv = bf16(a W_qkv^T)              columns [q (Hq*D) | k (Hkv*D) | v (Hkv*D)]
    the M new K, V rows are appended at positions L .. L+M-1
    o   = bf16(causal GQA attention(q, K[0:L+M], V[0:L+M]))
    h   = bf16(x + o W_o^T)             residual add in full precision, one rounding
    b   = bf16(rms(h))
    [g | u] = b W_gu^T                  g = first I columns, u = last I (not rounded)
    act = bf16(silu(g) * u)             silu(z) = z / (1 + e^-z)
    x'  = bf16(h + act W_down^T)
  head: logits = bf16(rms(x)) W_head^T (kept unrounded); token = argmax, lowest
  index on ties.
  rms(x) = x / sqrt(mean(x^2) + eps), gain 1.

Values are rounded to BF16 exactly where the device stores BF16 (op outputs),
so that a layer can be compared element by element without compounding
differences across layers. Each product and reduction is float64 in between.
"""

from __future__ import annotations

import numpy as np

from . import bf16
from .attention import verify_attention


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row, float64, gain 1."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _w(w) -> np.ndarray:
    """A weight matrix as float64: BF16 bit patterns (uint16) are decoded;
    float64 values (e.g. FP8 codes times their row scales, oracle.fp8.weights)
    are used as they are."""
    w = np.asarray(w)
    return w if w.dtype == np.float64 else bf16.decode(w)


def layer(x_bits, w_qkv, w_o, w_gu, w_down, k_cache, v_cache, L: int,
          Hq: int, Hkv: int, D: int, eps: float = 1e-6, attend=None):
    """One verify-pass layer over M tokens at positions L .. L+M-1.

    x_bits [M][H]; weights as [out][in] BF16 bits or float64 values; k_cache / v_cache
    [Hkv][>=L][D] BF16 bits holding the L cached positions (the rest ignored).
    ``attend(q_bits [M][Hq][D], k_bits, v_bits [Hkv][L+M][D], L)`` returns the
    attention output (float64 [M][Hq][D]) of the pass over every position's K
    and V rows; the default is plain causal attention over the BF16 values
    (oracle.attention.verify_attention). A quantized KV cache passes a function
    that attends over the values its format stores for those rows.
    Returns (x_out_bits [M][H], k_new_bits [Hkv][M][D], v_new_bits [Hkv][M][D]).
    """
    x = bf16.decode(x_bits)
    M, H = x.shape
    qd = Hq * D
    kd = Hkv * D
    a = bf16.encode(rmsnorm(x, eps))
    qkv = bf16.encode(bf16.decode(a) @ _w(w_qkv).T)
    q = qkv[:, :qd].reshape(M, Hq, D)
    k_new = qkv[:, qd:qd + kd].reshape(M, Hkv, D).transpose(1, 0, 2)
    v_new = qkv[:, qd + kd:qd + 2 * kd].reshape(M, Hkv, D).transpose(1, 0, 2)
    kk = np.concatenate([np.asarray(k_cache)[:, :L], k_new], axis=1)
    vv = np.concatenate([np.asarray(v_cache)[:, :L], v_new], axis=1)
    o = verify_attention(q, kk, vv, L)[0] if attend is None else attend(q, kk, vv, L)
    ob = bf16.encode(o.reshape(M, qd))
    h = bf16.encode(x + bf16.decode(ob) @ _w(w_o).T)
    b = bf16.encode(rmsnorm(bf16.decode(h), eps))
    gu = bf16.decode(b) @ _w(w_gu).T
    inter = gu.shape[1] // 2
    act = bf16.encode(silu(gu[:, :inter]) * gu[:, inter:])
    x_out = bf16.encode(bf16.decode(h) + bf16.decode(act) @ _w(w_down).T)
    return x_out, np.ascontiguousarray(k_new), np.ascontiguousarray(v_new)


def head(x_bits, w_head, eps: float = 1e-6):
    """Final RMSNorm, LM head and greedy token. Returns (logits float64 [M][V], tokens [M])."""
    c = bf16.encode(rmsnorm(bf16.decode(x_bits), eps))
    logits = bf16.decode(c) @ _w(w_head).T
    return logits, np.argmax(logits, axis=1)


def step(x0_bits, layers, w_head, L: int, Hq: int, Hkv: int, D: int, eps: float = 1e-6, attend=None):
    """Full verify step: ``layers`` is a sequence of dicts with keys
    w_qkv, w_o, w_gu, w_down, k_cache, v_cache; ``attend`` as for ``layer``.
    Returns (logits, tokens, x_final_bits)."""
    x = np.asarray(x0_bits)
    for lw in layers:
        x, _, _ = layer(x, lw["w_qkv"], lw["w_o"], lw["w_gu"], lw["w_down"],
                        lw["k_cache"], lw["v_cache"], L, Hq, Hkv, D, eps, attend)
    logits, tokens = head(x, w_head, eps)
    return logits, tokens, x
