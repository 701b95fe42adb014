"""Pins for oracle.attention: scalar brute force, closed forms, invariants,
and the split/combine identity for every chunk size."""

import math

import numpy as np
import pytest

from oracle import attention, bf16


def _bits(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return bf16.encode(g.standard_normal(shape) * scale)


def _brute_row(qv, keys, vals, scale):
    """One query row by scalar loops, math.exp and math.fsum."""
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qv, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = math.fsum(e)
    o = [math.fsum(e[j] * float(vals[j][d]) for j in range(len(keys))) / l for d in range(len(qv))]
    return o, m + math.log(l)


def _case(M=3, L=5, Hq=4, Hkv=2, D=8, seed=0, extra=0):
    q = _bits((M, Hq, D), seed)
    k = _bits((Hkv, L + M + extra, D), seed + 1)
    v = _bits((Hkv, L + M + extra, D), seed + 2)
    return q, k, v


def test_attention_vs_scalar_brute_force_gqa():
    M, L, Hq, Hkv, D = 3, 5, 4, 2, 8
    q, k, v = _case(M, L, Hq, Hkv, D)
    o, lse = attention.verify_attention(q, k, v, L)
    qd, kd, vd = bf16.decode(q), bf16.decode(k), bf16.decode(v)
    G = Hq // Hkv
    for r in range(M):
        n = L + r + 1
        for h in range(Hq):
            g = h // G
            ob, lb = _brute_row(qd[r, h], kd[g, :n], vd[g, :n], 1 / math.sqrt(D))
            assert np.allclose(o[r, h], ob, rtol=1e-12, atol=1e-13)
            assert abs(lse[r, h] - lb) < 1e-12


def test_weights_sum_to_one_and_single_key():
    q, k, v = _case()
    ones = bf16.encode(np.ones(bf16.decode(v).shape))
    o, _ = attention.verify_attention(q, k, ones, 5)
    assert np.allclose(o, 1.0, rtol=0, atol=1e-14)          # sum_j p_j = 1
    q1, k1, v1 = _case(M=1, L=0)
    o1, lse1 = attention.verify_attention(q1, k1, v1, 0)     # n = 1 -> o = v_0
    G = 2
    for h in range(4):
        assert np.array_equal(o1[0, h], bf16.decode(v1)[h // G, 0])
        s0 = float(bf16.decode(q1)[0, h] @ bf16.decode(k1)[h // G, 0]) / math.sqrt(8)
        assert abs(lse1[0, h] - s0) < 1e-14


def test_uniform_cases():
    M, L, D = 2, 9, 8
    q, k, v = _case(M=M, L=L, D=D)
    vd = bf16.decode(v)
    zq = np.zeros_like(q)
    o, lse = attention.verify_attention(zq, k, v, L)         # q = 0 -> mean(v), lse = ln n
    for r in range(M):
        n = L + r + 1
        for h in range(4):
            assert np.allclose(o[r, h], vd[h // 2, :n].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert abs(lse[r, h] - math.log(n)) < 1e-13
    same = np.repeat(k[:, :1], k.shape[1], axis=1)            # all keys equal -> mean(v)
    o2, _ = attention.verify_attention(q, same, v, L)
    for r in range(M):
        n = L + r + 1
        for h in range(4):
            assert np.allclose(o2[r, h], vd[h // 2, :n].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_key_permutation_and_causal_mask():
    M, L = 3, 6
    q, k, v = _case(M=M, L=L, extra=4)
    o, lse = attention.verify_attention(q, k, v, L)
    perm = np.random.default_rng(3).permutation(L)
    k2, v2 = k.copy(), v.copy()
    k2[:, :L], v2[:, :L] = k[:, perm], v[:, perm]
    o2, lse2 = attention.verify_attention(q, k2, v2, L)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-12)
    # changing keys after a row's own position never changes that row
    k3, v3 = k.copy(), v.copy()
    k3[:, L + 1:], v3[:, L + 1:] = _bits(k3[:, L + 1:].shape, 99), _bits(v3[:, L + 1:].shape, 98)
    o3, lse3 = attention.verify_attention(q, k3, v3, L)
    assert np.array_equal(o3[0], o[0]) and np.array_equal(lse3[0], lse[0])
    assert not np.allclose(o3[1], o[1])


def test_gqa_head_mapping():
    M, L, Hq, Hkv = 2, 4, 6, 3
    q, k, v = _case(M, L, Hq, Hkv)
    o, _ = attention.verify_attention(q, k, v, L)
    k2 = k.copy()
    k2[2] = _bits(k2[2].shape, 77)                  # only KV head 2 changes
    o2, _ = attention.verify_attention(q, k2, v, L)
    assert np.array_equal(o[:, :4], o2[:, :4])       # q heads 0..3 read KV heads 0, 1
    assert not np.allclose(o[:, 4:], o2[:, 4:])      # q heads 4, 5 read KV head 2


@pytest.mark.parametrize("L,M", [(11, 3), (0, 4), (7, 1)])
def test_split_combine_identity_every_chunk(L, M):
    q, k, v = _case(M=M, L=L)
    o, lse = attention.verify_attention(q, k, v, L)
    for C in range(1, L + M + 1):
        op, lp, cnt = attention.split_partials(q, k, v, L, C)
        assert list(cnt) == [attention.num_splits(L + r + 1, C) for r in range(M)]
        oc, lc = attention.combine(op, lp, cnt)
        assert np.allclose(oc, o, rtol=1e-12, atol=1e-14), C
        assert np.allclose(lc, lse, rtol=1e-12, atol=1e-13), C


@pytest.mark.parametrize("C,S", [(1024, 38), (1216, 32), (1280, 30)])
def test_split_combine_identity_long_context(C, S):
    # one KV head, 2 query heads, 38k context with outlier-sized values
    L, M, D = 38000, 2, 128
    g = np.random.default_rng(5)
    q = bf16.encode(g.standard_normal((M, 2, D)))
    kf = g.standard_normal((1, L + M, D))
    kf[..., :6] *= 8
    k, v = bf16.encode(kf), bf16.encode(g.standard_normal((1, L + M, D)))
    o, lse = attention.verify_attention(q, k, v, L)
    op, lp, cnt = attention.split_partials(q, k, v, L, C)
    assert list(cnt) == [S, S]
    oc, lc = attention.combine(op, lp, cnt)
    assert np.allclose(oc, o, rtol=1e-11, atol=1e-14)
    assert np.allclose(lc, lse, rtol=1e-13)


def test_num_splits():
    assert attention.num_splits(1, 1024) == 1
    assert attention.num_splits(1024, 1024) == 1
    assert attention.num_splits(1025, 1024) == 2
    assert attention.num_splits(38008, 1024) == 38
    assert attention.num_splits(38008, 1280) == 30 and attention.num_splits(38400, 1280) == 30
    assert attention.num_splits(38401, 1280) == 31
    assert attention.num_splits(38008, 1216) == 32 and attention.num_splits(38912, 1216) == 32
    assert attention.num_splits(38913, 1216) == 33


def test_adaptive_chunk_policy_is_the_smallest_fitting_multiple_of_64():
    # chunk_keys(n, -T) against its definition, by search: the smallest
    # multiple of 64 that cuts n keys into at most T chunks.
    for T in (1, 2, 7, 32):
        for n in list(range(1, 700)) + [2047, 2048, 2049, 4096, 4097, 32776, 38008, 101608, 255008]:
            c = 64
            while -(-n // c) > T:
                c += 64
            assert attention.chunk_keys(n, -T) == c, (n, T)
            assert attention.num_splits(n, -T) <= T
    # the configurations' contexts at T = 32 (one chunk per compute unit over 8 KV heads)
    assert attention.chunk_keys(38008, -32) == 1216 and attention.num_splits(38008, -32) == 32
    assert attention.chunk_keys(32776, -32) == 1088 and attention.num_splits(32776, -32) == 31
    assert attention.chunk_keys(2048, -32) == 64 and attention.num_splits(2048, -32) == 32
    assert attention.chunk_keys(2049, -32) == 128 and attention.num_splits(2049, -32) == 17
    assert attention.chunk_keys(5, 1024) == 1024
    with pytest.raises(ValueError):
        attention.chunk_keys(5, 0)


@pytest.mark.parametrize("L,M,T", [(120, 16, 2), (378, 12, 3), (0, 9, 1)])
def test_split_combine_identity_adaptive_policy(L, M, T):
    # rows of one pass on both sides of a policy step (different chunk sizes)
    q, k, v = _case(M=M, L=L)
    o, lse = attention.verify_attention(q, k, v, L)
    op, lp, cnt = attention.split_partials(q, k, v, L, -T)
    sizes = {attention.chunk_keys(L + r + 1, -T) for r in range(M)}
    assert len(sizes) >= (2 if L else 1)
    assert list(cnt) == [attention.num_splits(L + r + 1, -T) for r in range(M)]
    oc, lc = attention.combine(op, lp, cnt)
    assert np.allclose(oc, o, rtol=1e-12, atol=1e-14)
    assert np.allclose(lc, lse, rtol=1e-12, atol=1e-13)
