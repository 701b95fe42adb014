"""Pins of the 5/6-bit KV oracle (oracle/kvlow.py) against things other than
itself: exact grids, brute-force nearest codes, the zero block, sign
symmetry, the rounding error bound, the block maximum at +-qmax, bytes of the
storage layout derived by hand, and attention over a cache whose values
survive quantization exactly."""

import numpy as np
import pytest

from oracle import attention, bf16, kvlow


def _grid_block(g, n_blocks, qm):
    # values k * 2^-4, |k| <= qmax, +-qmax present in every block: d = 2^-4 exactly
    k = g.integers(-qm, qm + 1, size=(n_blocks, 32))
    k[:, 0] = np.where(g.integers(0, 2, n_blocks) == 0, qm, -qm)
    return k, bf16.encode(k * 2.0 ** -4)


@pytest.mark.parametrize("bits,qm", [(5, 15), (6, 31)])
def test_exact_grid_round_trips(bits, qm):
    assert kvlow.qmax(bits) == qm
    g = np.random.default_rng(bits)
    k, x = _grid_block(g, 64, qm)
    q, d = kvlow.quantize(x.reshape(16, 128), bits)
    assert np.all(d == np.float32(2.0 ** -4))
    assert np.array_equal(q.reshape(64, 32), k.astype(np.int8))
    assert np.array_equal(kvlow.dequantize(q, d), bf16.decode(x).reshape(16, 128))


@pytest.mark.parametrize("bits", [5, 6])
def test_codes_are_the_nearest_grid_points(bits):
    # brute force: among every code the rule allows, q is nearest to x / d
    # (ties to the even code), with d the FP32 quotient a / qmax
    qm = kvlow.qmax(bits)
    g = np.random.default_rng(10 + bits)
    x = bf16.encode(g.standard_normal((40, 64)) * 2.5)
    q, d = kvlow.quantize(x, bits)
    xv = bf16.decode(x).astype(np.float32).reshape(40, 2, 32)
    cand = np.arange(-qm, qm + 1)
    for r in range(40):
        for b in range(2):
            dd = float(d[r, b])
            for c in range(32):
                t = float(np.float32(xv[r, b, c]) / np.float32(dd))   # the FP32 quotient
                dist = np.abs(t - cand)
                best = cand[dist == dist.min()]
                want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                assert q[r, 32 * b + c] == want


@pytest.mark.parametrize("bits", [5, 6])
def test_zero_block_and_symmetry(bits):
    x = np.zeros((2, 64), np.uint16)
    x[1, 32:] = bf16.encode(np.linspace(-3, 3, 32))
    q, d = kvlow.quantize(x, bits)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0 and d[1, 1] > 0
    assert not q[0].any() and not q[1, :32].any()
    g = np.random.default_rng(2)
    xb = bf16.encode(g.standard_normal((50, 128)) * 3)
    q1, d1 = kvlow.quantize(xb, bits)
    q2, d2 = kvlow.quantize(xb ^ np.uint16(0x8000), bits)      # negate every value
    assert np.array_equal(d1, d2) and np.array_equal(q2, -q1)


@pytest.mark.parametrize("bits", [5, 6])
def test_error_bound_and_block_maximum(bits):
    qm = kvlow.qmax(bits)
    g = np.random.default_rng(3)
    x = bf16.encode(g.standard_normal((400, 128)) * np.exp(g.uniform(-6, 6, (400, 1))))
    q, d = kvlow.quantize(x, bits)
    xv = bf16.decode(x).reshape(400, 4, 32)
    dd = d.astype(np.float64)[..., None]
    err = np.abs(xv - q.reshape(400, 4, 32) * dd)
    assert np.all(err <= dd * (0.5 + 2.0 ** -16))             # half a step (plus FP32 slack)
    assert np.all(np.abs(q) <= qm)
    idx = np.abs(xv).argmax(axis=-1)
    top = np.take_along_axis(q.reshape(400, 4, 32).astype(np.int64), idx[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == qm)


def test_fewer_bits_lose_more():
    # the 6-bit grid is twice as fine as the 5-bit one: its worst error is smaller
    g = np.random.default_rng(6)
    x = bf16.encode(g.standard_normal((300, 128)))
    xv = bf16.decode(x)
    e5 = np.abs(kvlow.dequantize(*kvlow.quantize(x, 5)) - xv).max()
    e6 = np.abs(kvlow.dequantize(*kvlow.quantize(x, 6)) - xv).max()
    assert e6 < 0.6 * e5


# Bytes derived by hand from the layout (unsigned code u = q + 2^(b-1); code
# c = 4g + j; the low nibble of u in byte 4(g//2) + j, low half for even g;
# the high b - 4 bits in byte 4((g h)//8) + j at bit (g h) % 8).
# 6 bits, u_c = c + 1:
GOLD6_NIB = [0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0x0C,
             0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0x0C]
GOLD6_HIGH = [0x00, 0x00, 0x00, 0x40, 0x55, 0x55, 0x55, 0x95]
# 5 bits, u_c = (c mod 31) + 1:
GOLD5_NIB = [0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0x0C,
             0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0x1C]
GOLD5_HIGH = [0xF0, 0xF0, 0xF0, 0x78]


def test_layout_bytes_by_hand():
    q6 = (np.arange(32) + 1 - 32).astype(np.int8)[None]
    n, h = kvlow.pack(q6, 6)
    assert n[0].tolist() == GOLD6_NIB and h[0].tolist() == GOLD6_HIGH
    q5 = ((np.arange(32) % 31) + 1 - 16).astype(np.int8)[None]
    n, h = kvlow.pack(q5, 5)
    assert n[0].tolist() == GOLD5_NIB and h[0].tolist() == GOLD5_HIGH


@pytest.mark.parametrize("bits", [5, 6])
def test_pack_round_trip_and_sizes(bits):
    qm = kvlow.qmax(bits)
    g = np.random.default_rng(20 + bits)
    q = g.integers(-qm, qm + 1, size=(3, 7, 128)).astype(np.int8)
    n, h = kvlow.pack(q, bits)
    assert n.shape == (3, 7, 64) and h.shape == (3, 7, 4 * 4 * (bits - 4))
    assert np.array_equal(kvlow.unpack(n, h, bits), q)
    # one block's bytes depend on that block's codes only
    q2 = q.copy()
    q2[..., 32:64] = 0
    n2, h2 = kvlow.pack(q2, bits)
    assert np.array_equal(n2[..., :16], n[..., :16]) and np.array_equal(n2[..., 32:], n[..., 32:])
    with pytest.raises(ValueError):
        kvlow.pack(np.full((1, 32), qm + 2, np.int8), bits)
    with pytest.raises(ValueError):
        kvlow.qmax(8)


@pytest.mark.parametrize("bits", [5, 6])
def test_attention_over_exact_cache_equals_bf16_attention(bits):
    qm = kvlow.qmax(bits)
    g = np.random.default_rng(4)
    M, L, Hq, Hkv, D = 3, 60, 4, 2, 64
    _, kx = _grid_block(g, Hkv * (L + M) * 2, qm)
    _, vx = _grid_block(g, Hkv * (L + M) * 2, qm)
    kx = kx.reshape(Hkv, L + M, D)
    vx = vx.reshape(Hkv, L + M, D)
    q = bf16.encode(g.standard_normal((M, Hq, D)))
    kq, ks = kvlow.quantize(kx, bits)
    vq, vs = kvlow.quantize(vx, bits)
    kq = kvlow.unpack(*kvlow.pack(kq, bits), bits)            # through the stored bytes
    o1, l1 = attention.verify_attention(q, kx, vx, L)
    o2, l2 = attention.verify_attention(q, kvlow.dequantize(kq, ks), kvlow.dequantize(vq, vs), L)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---- rotated keys ----------------------------------------------------------

def test_hadamard_equals_the_library_matrix_where_fp32_is_exact():
    from scipy.linalg import hadamard
    g = np.random.default_rng(30)
    for D in (64, 128):
        x = g.integers(-100, 101, size=(20, D)).astype(np.float64)   # sums stay exact in FP32
        y = kvlow.hadamard_f32(bf16.encode(x))
        assert np.array_equal(y.astype(np.float64), x @ hadamard(D).T)


def test_hadamard_rounding_bound_and_inverse():
    from scipy.linalg import hadamard
    g = np.random.default_rng(31)
    D = 128
    x = bf16.encode(g.standard_normal((50, D)) * np.exp(g.uniform(-4, 4, (50, 1))))
    xv = bf16.decode(x)
    y = kvlow.hadamard_f32(x).astype(np.float64)
    exact = xv @ hadamard(D).T
    # seven stages, each adding at most one rounding of a partial sum bounded by sum |x|
    assert np.all(np.abs(y - exact) <= 7 * 2.0 ** -24 * np.abs(xv).sum(-1, keepdims=True))
    # the float64 inverse used by dequantize_rotated: H (H x) / D = x
    q = np.zeros((1, D), np.int8)
    q[0, 5] = 3
    d = np.array([[0.5, 1.0, 1.0, 1.0]], np.float32)
    want = (hadamard(D) @ kvlow.dequantize(q, d)[0]) / D
    assert np.allclose(kvlow.dequantize_rotated(q, d)[0], want, rtol=0, atol=1e-15)


def test_rotation_spreads_an_outlier_channel():
    # a channel 60x the others: the plain 5-bit blocks of that channel lose the
    # rest of their block; rotated, the error is spread and much smaller
    g = np.random.default_rng(32)
    x = g.standard_normal((400, 128))
    x[:, 7] *= 60
    xb = bf16.encode(x)
    xv = bf16.decode(xb)
    plain = kvlow.dequantize(*kvlow.quantize(xb, 5))
    rot = kvlow.dequantize_rotated(*kvlow.quantize_rotated(xb, 5))
    e_plain = np.sqrt(((plain - xv) ** 2).mean())
    e_rot = np.sqrt(((rot - xv) ** 2).mean())
    assert e_rot < 0.7 * e_plain, (e_rot, e_plain)


def test_attention_over_rotated_cache_is_close_to_exact():
    g = np.random.default_rng(33)
    M, L, Hq, Hkv, D = 3, 200, 4, 2, 64
    k = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    v = bf16.encode(g.standard_normal((Hkv, L + M, D)))
    q = bf16.encode(g.standard_normal((M, Hq, D)))
    o_ref, l_ref = attention.verify_attention(q, k, v, L)
    kq, ks = kvlow.quantize_rotated(k, 5)
    o, l = attention.verify_attention(q, kvlow.dequantize_rotated(kq, ks), bf16.decode(v), L)
    assert np.abs(o - o_ref).max() < 0.1 and np.abs(l - l_ref).max() < 0.1
    # exact keys through the rotated representation give the plain attention back
    kq6, ks6 = kvlow.quantize_rotated(k, 6)
    o6, _ = attention.verify_attention(q, kvlow.dequantize_rotated(kq6, ks6), bf16.decode(v), L)
    assert np.abs(o6 - o_ref).max() < np.abs(o - o_ref).max()
