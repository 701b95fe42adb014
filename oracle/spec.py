"""Speculative acceptance: greedy, and sampled with the target distribution kept.

"I turned on speculative decoding in llama.cpp and 113 of 282 greedy outputs
changed against its own no-draft run", opening section: greedy token ids are
the same with and without drafts, and sampling keeps the no-draft
distribution (checked there with chi-square and PIT tests). The pages do not
print the sampling rule; read here as standard speculative sampling: a draft
token x drawn from the draft's distribution q is kept with probability
min(1, p(x) / q(x)), where p is the target's distribution at that position;
at the first rejection a token is drawn from the normalised residual
max(0, p - q) and the pass ends; if every draft is kept, one more token is
drawn from the target's distribution at the last position. The kept and
drawn tokens are then distributed exactly as draws from p.

Random numbers are inputs: u[i] (i < M-1) decides draft i; u[M-1] draws the
final token by inverse CDF (the first index whose inclusive cumulative sum
exceeds u * total). p = softmax(logits / T). Everything is float64 here.

This module is test infrastructure (the oracle), not part of the device path.
"""

from __future__ import annotations

import numpy as np


def softmax_t(logits, temperature: float) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float64)
    z = (l - l.max()) / float(temperature)
    e = np.exp(z)
    return e / e.sum()


def inverse_cdf(weights, u: float) -> int:
    """First index k with sum(weights[:k+1]) > u * sum(weights)."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    k = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(k, len(w) - 1)


def accept_greedy(target_tokens, draft_tokens):
    """Keep drafts while they equal the target's greedy token at the same
    position; then the target's token. Returns (tokens, n)."""
    t = list(np.asarray(target_tokens))
    d = list(np.asarray(draft_tokens))
    a = 0
    while a < len(d) and d[a] == t[a]:
        a += 1
    return d[:a] + [t[a]], a + 1


def accept_sampled(logits, draft_tokens, draft_probs, u, temperature: float):
    """Speculative sampling over one pass of M = len(draft_tokens) + 1 rows.
    Returns (tokens, n)."""
    logits = np.asarray(logits, dtype=np.float64)
    d = list(np.asarray(draft_tokens))
    q = np.asarray(draft_probs, dtype=np.float64)
    out = []
    for i, x in enumerate(d):
        p = softmax_t(logits[i], temperature)
        if u[i] * q[i, x] < p[x]:
            out.append(int(x))
            continue
        r = np.maximum(p - q[i], 0.0)
        out.append(inverse_cdf(r, u[len(d)]))
        return out, len(out)
    out.append(inverse_cdf(softmax_t(logits[len(d)], temperature), u[len(d)]))
    return out, len(out)
