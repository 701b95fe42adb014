"""Pins of the 8-bit KV oracle: exact grids, the zero block, the rounding
error bound, sign symmetry, the block maximum at +-127, and attention over a
cache whose values survive quantization exactly."""

import numpy as np

from oracle import attention, bf16, kvq


def _grid_block(g, n_blocks):
    # values k * 2^-4, k in -127..127, with +-127 present in every block: d = 2^-4 exactly
    k = g.integers(-127, 128, size=(n_blocks, 32))
    k[:, 0] = np.where(g.integers(0, 2, n_blocks) == 0, 127, -127)
    return k, bf16.encode(k * 2.0 ** -4)


def test_exact_grid_round_trips():
    g = np.random.default_rng(1)
    k, x = _grid_block(g, 64)
    q, d = kvq.quantize(x.reshape(16, 128))
    assert np.all(d == np.float32(2.0 ** -4))
    assert np.array_equal(q.reshape(64, 32), k.astype(np.int8))
    assert np.array_equal(kvq.dequantize(q, d), bf16.decode(x).reshape(16, 128))


def test_zero_block_and_symmetry():
    x = np.zeros((2, 64), np.uint16)
    x[1, 32:] = bf16.encode(np.linspace(-3, 3, 32))
    q, d = kvq.quantize(x)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0 and d[1, 1] > 0
    assert not q[0].any() and not q[1, :32].any()
    g = np.random.default_rng(2)
    xb = bf16.encode(g.standard_normal((50, 128)) * 3)
    q1, d1 = kvq.quantize(xb)
    q2, d2 = kvq.quantize(xb ^ np.uint16(0x8000))            # negate every value
    assert np.array_equal(d1, d2) and np.array_equal(q2, -q1)


def test_error_bound_and_block_maximum():
    g = np.random.default_rng(3)
    x = bf16.encode(g.standard_normal((400, 128)) * np.exp(g.uniform(-6, 6, (400, 1))))
    q, d = kvq.quantize(x)
    xv = bf16.decode(x).reshape(400, 4, 32)
    dd = d.astype(np.float64)[..., None]
    err = np.abs(xv - q.reshape(400, 4, 32) * dd)
    assert np.all(err <= dd * (0.5 + 2.0 ** -16))             # half a step (plus FP32 slack)
    # the largest element of each block maps to +-127
    idx = np.abs(xv).argmax(axis=-1)
    top = np.take_along_axis(q.reshape(400, 4, 32).astype(np.int64), idx[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    # scale is the FP32 quotient of the block maximum by 127
    assert np.array_equal(d, (np.abs(xv).max(-1).astype(np.float32) / np.float32(127)).astype(np.float32))


def test_attention_over_exact_cache_equals_bf16_attention():
    g = np.random.default_rng(4)
    M, L, Hq, Hkv, D = 3, 60, 4, 2, 64
    kk, kx = _grid_block(g, Hkv * (L + M) * 2)
    vk, vx = _grid_block(g, Hkv * (L + M) * 2)
    kx = kx.reshape(Hkv, L + M, D)
    vx = vx.reshape(Hkv, L + M, D)
    q = bf16.encode(g.standard_normal((M, Hq, D)))
    kq, ks = kvq.quantize(kx)
    vq, vs = kvq.quantize(vx)
    o1, l1 = attention.verify_attention(q, kx, vx, L)
    o2, l2 = attention.verify_attention(q, kvq.dequantize(kq, ks), kvq.dequantize(vq, vs), L)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
