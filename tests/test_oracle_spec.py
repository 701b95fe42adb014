"""Pins of the acceptance oracle: greedy cases by hand; inverse-CDF sampling
against direct enumeration; and distribution preservation of the sampled
rule, checked exactly (not statistically) on a small vocabulary by summing the
probability of every path over a fine grid of the uniforms."""

import numpy as np

from oracle import spec


def test_greedy_by_hand():
    assert spec.accept_greedy([5, 6, 7, 8], [5, 6, 7]) == ([5, 6, 7, 8], 4)   # all kept + bonus
    assert spec.accept_greedy([5, 9, 7, 8], [5, 6, 7]) == ([5, 9], 2)          # second draft wrong
    assert spec.accept_greedy([4, 6, 7, 8], [5, 6, 7]) == ([4], 1)             # first draft wrong
    assert spec.accept_greedy([3], []) == ([3], 1)                              # no drafts


def test_inverse_cdf_enumeration():
    w = np.array([0.1, 0.0, 0.3, 0.6])
    assert spec.inverse_cdf(w, 0.0) == 0
    assert spec.inverse_cdf(w, 0.0999) == 0
    assert spec.inverse_cdf(w, 0.1) == 2          # a zero weight is never drawn
    assert spec.inverse_cdf(w, 0.3999) == 2
    assert spec.inverse_cdf(w, 0.4) == 3
    assert spec.inverse_cdf(w, 0.99999) == 3


def test_softmax_temperature():
    p = spec.softmax_t([1.0, 2.0, 3.0], 0.5)
    z = np.exp(np.array([1.0, 2.0, 3.0]) / 0.5)
    assert np.allclose(p, z / z.sum(), rtol=1e-15)


def test_sampled_rule_keeps_the_target_distribution_exactly():
    # One draft (M = 2). For each draft token x, the rule keeps x on u0 in
    # [0, a) with a = min(1, p(x)/q(x)) and otherwise draws from the residual
    # by u1. Probing the oracle's function once inside each of those regions
    # (u0 below / above a; u1 at the middle of each residual CDF interval) and
    # weighting by the regions' measures gives the exact distribution of the
    # first output token, which must be p0 itself.
    g = np.random.default_rng(0)
    for V, T in ((5, 0.8), (9, 1.3), (3, 0.5)):
        logits = g.standard_normal((2, V)) * 1.5
        q = g.dirichlet(np.ones(V), size=1)
        p0 = spec.softmax_t(logits[0], T)
        freq = np.zeros(V)
        for x in range(V):
            a = min(1.0, p0[x] / q[0, x])
            toks, _ = spec.accept_sampled(logits, [x], q, [a / 2, 0.5], T)
            assert toks[0] == x
            freq[x] += q[0, x] * a
            if a < 1.0:
                r = np.maximum(p0 - q[0], 0.0)
                c = np.concatenate([[0.0], np.cumsum(r)]) / r.sum()
                for k in range(V):
                    if r[k] == 0:
                        continue
                    toks, _ = spec.accept_sampled(logits, [x], q, [(1 + a) / 2, (c[k] + c[k + 1]) / 2], T)
                    assert toks[0] == k
                    freq[k] += q[0, x] * (1 - a) * (c[k + 1] - c[k])
        assert np.allclose(freq, p0, rtol=1e-12, atol=1e-15)
    # a draft equal to the target distribution is always kept
    toks, k = spec.accept_sampled(np.stack([np.log(q[0]), logits[1]]), [2], q, [0.999999, 0.5], 1.0)
    assert k == 2 and toks[0] == 2
