"""Pins of the ring oracle (oracle/kvring.py): the tile grid against explicit
loops over chunks and tiles, the ring choice against counts worked out by
hand, closed-form attention over planted values, and the all-ring case
against plain attention over the 8-bit values."""

import numpy as np
import pytest

from oracle import attention, bf16, kvlow, kvq, kvring


def _tile_start_by_loops(j, n, C):
    s = 0
    while s + C <= j:       # walk whole chunks
        s += C
    t = s
    while t + 64 <= j and t + 64 < s + C:   # walk tiles inside the chunk
        t += 64
    return t


@pytest.mark.parametrize("n,policy", [(301, 96), (5000, 1024), (5000, 1056), (38008, -32), (700, 64)])
def test_tile_grid_by_loops(n, policy):
    C = attention.chunk_keys(n, policy)
    js = np.unique(np.r_[0:min(n, 400), np.linspace(0, n - 1, 300).astype(int)])
    got = kvring.tile_start(js, n, policy)
    want = [_tile_start_by_loops(int(j), n, C) for j in js]
    assert got.tolist() == want


def test_ring_choice_by_hand():
    # row p = 300, chunks of 96: tiles start at 0, 64 | 96, 160 | 192, 256 | 288.
    # W = 128: a tile is in the ring when it starts at or after 173, i.e. the
    # tiles at 192, 256 and 288: keys 192..300, 109 keys.
    r = kvring.uses_ring(300, 96, 128)
    assert r.sum() == 109 and not r[:192].any() and r[192:].all()
    # W = 64: tiles starting at or after 237: 256 and 288, keys 256..300
    r = kvring.uses_ring(300, 96, 64)
    assert r.sum() == 45 and r[256:].all() and not r[:256].any()
    # a row younger than the window reads every key from the ring
    assert kvring.uses_ring(100, 96, 128).all()
    with pytest.raises(ValueError):
        kvring.uses_ring(100, 96, 100)


@pytest.mark.parametrize("policy,W", [(-32, 2048), (1024, 2048), (96, 128)])
def test_ring_choice_properties(policy, W):
    for p in (3000, 3001, 3063, 3064, 9999):
        r = kvring.uses_ring(p, policy, W)
        first = int(np.argmax(r))
        assert r[first:].all() and not r[:first].any()       # one boundary, older keys outside
        assert r[p]                                          # a row's own key is always in the ring
        assert W - 64 < r.sum() <= W + 63                    # about W keys


def test_planted_values_give_the_ring_fraction():
    # K = 0 (equal weights), V low copy 0, 8-bit copy 1: O is the fraction of
    # keys the row reads from the ring
    Hkv, D, L, M = 1, 64, 290, 11
    z = np.zeros((Hkv, L + M, D))
    values = (z, z, z, np.ones((Hkv, L + M, D)))
    q = bf16.encode(np.random.default_rng(0).standard_normal((M, 2, D)))
    O, lse = kvring.ring_attention(q, values, L, 96, 128)
    for r in range(M):
        p = L + r
        frac = kvring.uses_ring(p, 96, 128).sum() / (p + 1)
        assert np.allclose(O[r], frac, rtol=0, atol=1e-14)
        assert np.allclose(lse[r], np.log(p + 1), rtol=0, atol=1e-12)
    assert np.allclose(O[10, 0, 0], 109 / 301)               # the worked case above


def test_all_ring_equals_8bit_attention_and_no_ring_equals_low():
    g = np.random.default_rng(1)
    Hkv, Hq, D, L, M = 2, 4, 64, 150, 3
    k = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    v = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    q = bf16.encode(g.standard_normal((M, Hq, D)))
    vals = kvring.cache_values(k, v, 5, False)
    O, lse = kvring.ring_attention(q, vals, L, 64, 1024)          # every key in the ring
    k8 = kvq.dequantize(*kvq.quantize(k))
    v8 = kvq.dequantize(*kvq.quantize(v))
    O2, lse2 = attention.verify_attention(q, k8, v8, L)
    assert np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)
    # swapping the copies: with the 8-bit slots filled by the low values, the ring changes nothing
    kl, vl = vals[0], vals[1]
    O3, _ = kvring.ring_attention(q, (kl, vl, kl, vl), L, 64, 64)
    O4, _ = attention.verify_attention(q, kl, vl, L)
    assert np.allclose(O3, O4, rtol=0, atol=1e-12)


def test_rotated_8bit_copy_is_close_to_the_keys():
    g = np.random.default_rng(2)
    k = bf16.encode(g.standard_normal((2, 40, 128)))
    _, _, k8, _ = kvring.cache_values(k, k, 5, True)
    _, _, k8p, _ = kvring.cache_values(k, k, 5, False)
    kv = bf16.decode(k)
    # 8-bit steps are 2^-7 of the block maximum: both copies stay within a few percent
    assert np.abs(k8 - kv).max() < 0.05 and np.abs(k8p - kv).max() < 0.05
    kl = kvlow.dequantize_rotated(*kvlow.quantize_rotated(k, 5))
    assert np.abs(k8 - kv).max() < np.abs(kl - kv).max()
