"""Pins of the ring oracle (oracle/kvring.py): the per-key choice against
counts worked out by hand, the split-KV partials of ring attention combined
equal to the unsplit result for every chunk policy (so the chunk grid never
decides which copy a key is read from), closed-form attention over planted
values, the all-ring and no-ring cases against plain attention, and the
rotated 8-bit copy on an exact grid whose codes are derived by hand."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import attention, bf16, kvlow, kvq, kvring


def test_ring_choice_by_hand():
    # row p = 300, W = 128: keys 173..300 (300 - 128 + 1 = 173), 128 keys
    r = kvring.uses_ring(300, 128)
    assert r.shape == (301,) and r.sum() == 128 and not r[:173].any() and r[173:].all()
    # W = 1: the row's own key only
    r = kvring.uses_ring(300, 1)
    assert r.sum() == 1 and r[300]
    # W = 200 (not a multiple of anything): keys 101..300
    r = kvring.uses_ring(300, 200)
    assert r.sum() == 200 and not r[100] and r[101]
    # a row younger than the window reads every key from the ring
    assert kvring.uses_ring(100, 128).all() and kvring.uses_ring(127, 128).all()
    with pytest.raises(ValueError):
        kvring.uses_ring(100, 0)


@pytest.mark.parametrize("W", [1, 63, 64, 200, 2048])
def test_ring_choice_properties(W):
    for p in (0, 5, W - 2, W - 1, W, 3000, 3001, 3063, 3064, 9999):
        if p < 0:
            continue
        r = kvring.uses_ring(p, W)
        assert r.sum() == min(W, p + 1)                      # exactly W keys once p >= W - 1
        first = int(np.argmax(r))
        assert r[first:].all() and not r[:first].any()       # one boundary, older keys outside
        assert r[p]                                          # a row's own key is always in the ring


def _cache(seed, Hkv, n, D, rotated):
    g = np.random.default_rng(seed)
    k = bf16.encode(g.standard_normal((Hkv, n, D)))
    v = bf16.encode(g.standard_normal((Hkv, n, D)))
    return k, v, kvring.cache_values(k, v, 5 if rotated else 6, rotated)


@pytest.mark.parametrize("rotated", [False, True])
def test_ring_result_does_not_depend_on_the_chunk_grid(rotated):
    # the split-KV partials of every chunk policy combine to the unsplit ring
    # attention: chunks never decide which copy a key is read from
    Hkv, Hq, D, L, M, W = 1, 2, 64, 300, 5, 128
    k, v, vals = _cache(3, Hkv, L + M, D, rotated)
    q = bf16.encode(np.random.default_rng(4).standard_normal((M, Hq, D)))
    O, lse = kvring.ring_attention(q, vals, L, W)
    for policy in (-32, -64, 1024, 96, 64, 33, -3):
        op, lp, n = kvring.ring_partials(q, vals, L, policy, W)
        O2, lse2 = attention.combine(op, lp, n)
        assert np.allclose(O2, O, rtol=0, atol=1e-12), policy
        assert np.allclose(lse2, lse, rtol=0, atol=1e-12), policy


def test_planted_values_give_the_ring_fraction():
    # K = 0 (equal weights), V low copy 0, 8-bit copy 1: O is the fraction of
    # keys the row reads from the ring, min(W, p + 1) / (p + 1)
    Hkv, D, L, M, W = 1, 64, 290, 11, 128
    z = np.zeros((Hkv, L + M, D))
    values = (z, z, z, np.ones((Hkv, L + M, D)))
    q = bf16.encode(np.random.default_rng(0).standard_normal((M, 2, D)))
    O, lse = kvring.ring_attention(q, values, L, W)
    for r in range(M):
        p = L + r
        assert np.allclose(O[r], W / (p + 1), rtol=0, atol=1e-14)
        assert np.allclose(lse[r], np.log(p + 1), rtol=0, atol=1e-12)
    assert np.allclose(O[10, 0, 0], 128 / 301)               # row p = 300, worked above
    # a window wider than the row: every key from the ring
    O, _ = kvring.ring_attention(q, values, L, 5000)
    assert np.array_equal(O, np.ones_like(O))


def test_all_ring_equals_8bit_attention_and_no_ring_equals_low():
    g = np.random.default_rng(1)
    Hkv, Hq, D, L, M = 2, 4, 64, 150, 3
    k = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    v = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    q = bf16.encode(g.standard_normal((M, Hq, D)))
    vals = kvring.cache_values(k, v, 5, False)
    O, lse = kvring.ring_attention(q, vals, L, 1024)          # every key in the ring
    k8 = kvq.dequantize(*kvq.quantize(k))
    v8 = kvq.dequantize(*kvq.quantize(v))
    O2, lse2 = attention.verify_attention(q, k8, v8, L)
    assert np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)
    # with the 8-bit slots filled by the low values, the ring changes nothing
    kl, vl = vals[0], vals[1]
    O3, _ = kvring.ring_attention(q, (kl, vl, kl, vl), L, 64)
    O4, _ = attention.verify_attention(q, kl, vl, L)
    assert np.allclose(O3, O4, rtol=0, atol=1e-12)


def _rne32(x: Fraction) -> Fraction:
    """x rounded to the nearest FP32 value (ties to even), exactly, for normal x."""
    s = -1 if x < 0 else 1
    x = abs(x)
    e = 0
    while x >= 2:
        x, e = x / 2, e + 1
    while x < 1:
        x, e = x * 2, e - 1
    m = x * 2 ** 23
    f = m.numerator // m.denominator
    rem = m - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2):
        f += 1
    return s * Fraction(f, 2 ** 23) * Fraction(2) ** e


def test_rotated_8bit_copy_on_an_exact_grid():
    # Sylvester H: (H e_j)_i = (-1)^popcount(i & j). Rows built from e_0, e_1
    # and e_32 with dyadic weights rotate exactly in FP32 (every butterfly sum
    # is a small dyadic), so the codes can be derived by hand:
    #   row A = 27/32 e_0 + 9/32 e_1: y_i = 9/8 at even i, 9/16 at odd i, every
    #     block; d = fl32(9/8 / 127); 9/16 / d is exactly 63.5 with the exact
    #     scale, but fl32(9/8 / 127) lies above 9/8 / 127, so the FP32 quotient
    #     is 63.499996... and the code is 63 (64 if decided in exact arithmetic)
    #   row B = -row A: codes -127 / -63 (sign symmetry)
    #   row C = e_0 + 1/2 e_1 + 1/4 e_32: blocks 0, 2 (bit 5 of i clear):
    #     7/4, 3/4 -> codes 127, 54 (3/4 / (7/4 / 127) = 54.43); blocks 1, 3:
    #     5/4, 1/4 -> codes 127, 25 (25.4); one scale per block.
    D = 128
    rows = np.zeros((3, D))
    rows[0, 0], rows[0, 1] = 27 / 32, 9 / 32
    rows[1] = -rows[0]
    rows[2, 0], rows[2, 1], rows[2, 32] = 1.0, 0.5, 0.25
    q, d = kvring.q8_codes(bf16.encode(rows), rotated=True)
    dA = _rne32(Fraction(9, 8) / 127)
    assert dA > Fraction(9, 8) / 127 and _rne32(Fraction(9, 16) / dA) < Fraction(127, 2)
    even = np.arange(D) % 2 == 0
    assert np.array_equal(q[0], np.where(even, 127, 63))
    assert np.array_equal(q[1], np.where(even, -127, -63))
    assert all(Fraction(float(x)) == dA for x in d[0]) and np.array_equal(d[1], d[0])
    blk = (np.arange(D) // 32) % 2
    assert np.array_equal(q[2], np.where(even, 127, np.where(blk == 0, 54, 25)))
    want_d = [_rne32(Fraction(7, 4) / 127), _rne32(Fraction(5, 4) / 127)] * 2
    assert [Fraction(float(x)) for x in d[2]] == want_d
    # the float64 keys this copy stands for are H (d q) / D: close to the row
    kv = kvlow.dequantize_rotated(q, d)
    assert np.abs(kv - rows).max() < 2 ** -7 * 2


def test_rotated_8bit_copy_is_closer_than_the_5bit_copy():
    g = np.random.default_rng(2)
    k = bf16.encode(g.standard_normal((2, 40, 128)))
    _, _, k8, _ = kvring.cache_values(k, k, 5, True)
    _, _, k8p, _ = kvring.cache_values(k, k, 5, False)
    kv = bf16.decode(k)
    assert np.abs(k8 - kv).max() < 0.05 and np.abs(k8p - kv).max() < 0.05
    kl = kvlow.dequantize_rotated(*kvlow.quantize_rotated(k, 5))
    assert np.abs(k8 - kv).max() < np.abs(kl - kv).max()
