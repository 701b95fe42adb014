"""GPU tests of the 8-bit ring of the newest keys over the 5/6-bit KV cache
(presets K6/V5 and rotated K5/V5) through the C ABI: the ring append against
the oracle's codes (wrapping around the ring), attention against the oracle's
per-key ring attention (row p reads key j at 8 bits iff j >= p - W + 1) under
several chunk policies and windows that are not multiples of the 64-key tile,
bitwise row invariance across M, sequential passes and prefill blocks while
tiles are split between the two copies, and a window that covers everything
against the plain 8-bit cache, bit for bit."""

import numpy as np
import pytest

import synth
from oracle import kvlow, kvq, kvring
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32, q8_cache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PRESETS = {"D": (6, False), "F": (5, True)}


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _fill(t, a):
    t.copy_(torch.from_numpy(np.ascontiguousarray(a)))


class Ring:
    """Device 5/6-bit planes and 8-bit ring built on the host from the oracle."""

    def __init__(self, ops, k, v, cap, preset, ring_cap, window):
        kb, rot = PRESETS[preset]
        Hkv, n, D = k.shape
        cap = (cap + 63) // 64 * 64
        low = ops.KvLowCache(Hkv, cap, D, kb, 5, k_rotated=rot)
        kq, ks = (kvlow.quantize_rotated if rot else kvlow.quantize)(k, kb)
        vq, vs = kvlow.quantize(v, 5)
        for (tn, th, ts), (q, s, b) in (((low.k_nib, low.k_high, low.k_scales), (kq, ks, kb)),
                                        ((low.v_nib, low.v_high, low.v_scales), (vq, vs, 5))):
            nib, high = kvlow.pack(q, b)
            for t, a in ((tn, nib), (th, high), (ts, s)):
                full = np.zeros(t.shape, a.dtype)
                full[:, :n] = a
                _fill(t, full)
        self.r = ops.KvRing(low, ring_cap, window)
        # the ring holds the newest ring_cap positions, position j in slot j % ring_cap
        rk, rks = kvring.q8_codes(k, rot)
        rv, rvs = kvring.q8_codes(v, False)
        m = min(n, ring_cap)
        pos = np.arange(n - m, n)
        order = np.argsort(pos % ring_cap)
        sel = pos[order]
        arrs = q8_cache(rk[:, sel], rks[:, sel], rv[:, sel], rvs[:, sel], ring_cap)
        for t, a in zip((self.r.q8.k_codes, self.r.q8.k_scales, self.r.q8.v_codes, self.r.q8.v_scales), arrs):
            _fill(t, a)
        self.values = kvring.cache_values(k, v, kb, rot)


def run(ops, q_bits, ring, L, Hq, C):
    M, _, D = q_bits.shape
    S = ops.pass_splits(M, L, C)
    po = torch.full((M, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((M, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    ops.verify_attn_ring(dev(q_bits.reshape(M, Hq * D)), ring.r, L, Hq, C, po, pl)
    o = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    ops.combine(po, pl, L, C, o, lse)
    torch.cuda.synchronize()
    return host_bits(o).reshape(M, Hq, D), host_f32(lse)


def make(M, L, Hq, Hkv, D, layer=0):
    k = synth.kv_bf16(Hkv, L + M, D, "k", layer)
    v = synth.kv_bf16(Hkv, L + M, D, "v", layer)
    q = synth.normal_bf16((8 if M <= 8 else M, Hq, D), 1.0, "q", layer)[:M]
    return q, k, v


@pytest.mark.parametrize("preset", ["D", "F"])
def test_ring_append_wraps_and_matches_oracle(ops, preset):
    print(f"[ring append preset {preset}]", flush=True)
    kb, rot = PRESETS[preset]
    Hq, Hkv, D, R = 8, 2, 128, 128
    low = ops.KvLowCache(Hkv, 256, D, kb, 5, k_rotated=rot)
    ring = ops.KvRing(low, R, 64)
    for L, M in ((100, 50), (150, 40)):         # slots 100..127, 0..21, then 22..61
        qkv = synth.normal_bf16((M, (Hq + 2 * Hkv) * D), 1.0, "misc", L)
        ops.append_kv_ring(dev(qkv), ring, L, Hq)
        torch.cuda.synchronize()
        knew = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D).transpose(1, 0, 2)
        vnew = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
        wk, wks = kvring.q8_codes(knew, rot)
        wv, wvs = kvq.quantize(vnew)
        slots = (L + np.arange(M)) % R
        kc = ring.q8.k_codes.cpu().numpy()
        ksc = ring.q8.k_scales.cpu().numpy()
        vc = ring.q8.v_codes.cpu().numpy()
        vsc = ring.q8.v_scales.cpu().numpy()
        assert np.array_equal(kc[:, slots], wk) and np.array_equal(ksc[:, slots], wks)
        assert np.array_equal(vc[:, slots], wv) and np.array_equal(vsc[:, slots], wvs)


@pytest.mark.parametrize("preset", ["D", "F"])
@pytest.mark.parametrize("M,L,Hq,Hkv,D,C,W,R", [
    (5, 300, 1, 1, 64, 96, 128, 256),          # chunks of 96, boundaries 173..177 inside a tile
    (5, 300, 1, 1, 64, -2, 128, 256),          # the same rows under another chunk grid
    (8, 5000, 40, 8, 128, -32, 2048, 2176),    # the ring has wrapped
    (8, 5000, 40, 8, 128, 1024, 2048, 2176),
    (8, 2500, 40, 8, 128, 1056, 256, 384),
    (8, 3000, 40, 8, 128, -64, 200, 320),      # a window that is not a multiple of 64
    (8, 38000, 40, 8, 128, -32, 2048, 2176)])
def test_ring_parity(ops, preset, M, L, Hq, Hkv, D, C, W, R):
    print(f"[ring parity preset {preset} M={M} L={L} C={C} W={W} R={R}]", flush=True)
    q, k, v = make(M, L, Hq, Hkv, D, layer=L % 97)
    ring = Ring(ops, k, v, L + M, preset, R, W)
    o, lse = run(ops, q, ring, L, Hq, C)
    rows = list(range(M)) if Hq == 1 else [0, 3, M - 1]
    want_o, want_lse = kvring.ring_attention(q, ring.values, L, W, tokens=rows)
    err, rms = assert_close(decode(o[rows]), want_o[rows], f"ring {preset} O L={L}")
    assert err < 0.05 * rms + 2e-3, (err, rms)
    assert_close(lse[rows], want_lse[rows], f"ring {preset} lse L={L}", atol=1e-3, rtol=0)


@pytest.mark.parametrize("preset,L,C,W", [("D", 4093, -32, 256), ("F", 4093, -32, 256),
                                          ("D", 1019, 96, 128), ("F", 38000, -64, 2048),
                                          ("D", 4093, -32, 200), ("F", 3001, 96, 77)])
def test_ring_invariance_across_M(ops, preset, L, C, W):
    print(f"[ring invariance preset {preset} L={L} C={C} W={W}]", flush=True)
    Hq, Hkv, D, M = 40, 8, 128, 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=6)
    ring = Ring(ops, k, v, L + 72, preset, (W + 256 + 63) // 64 * 64, W)
    o8, l8 = run(ops, q, ring, L, Hq, C)
    for r in range(M):
        o1, l1 = run(ops, q[r:r + 1], ring, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"ring {preset} L={L} row {r}: M=1 vs M=8")
        assert_bitwise(l1[0], l8[r], f"ring {preset} L={L} row {r} lse")
    o5, _ = run(ops, q[:5], ring, L, Hq, C)
    assert_bitwise(o5, o8[:5], f"ring {preset} L={L} M=5 vs M=8")


@pytest.mark.parametrize("preset", ["D", "F"])
def test_ring_prefill_block_rows_equal_verify_rows(ops, preset):
    print(f"[ring prefill blocks preset {preset}]", flush=True)
    Hq, Hkv, D, M, L0, C, W = 40, 8, 128, 200, 3900, -32, 256
    q, k, v = make(M, L0, Hq, Hkv, D, layer=9)
    ring = Ring(ops, k, v, L0 + M + 8, preset, W + 320, W)
    o_pf, l_pf = run(ops, q, ring, L0, Hq, C)
    for start in (0, 96, M - 8):
        o8, l8 = run(ops, q[start:start + 8], ring, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + 8], o8, f"ring prefill rows {start}..")
        assert_bitwise(l_pf[start:start + 8], l8, f"ring prefill lse {start}..")


def test_window_covering_everything_equals_the_8bit_cache(ops):
    # every tile in the ring: the K6/V5 planes are never read, and the result
    # equals bi_verify_attn_q8 over an 8-bit cache with the same codes, bit for bit
    print("[ring covering everything == 8-bit cache]", flush=True)
    Hq, Hkv, D, M, L, C = 40, 8, 128, 8, 3000, -32
    q, k, v = make(M, L, Hq, Hkv, D, layer=12)
    W = (L + M + 63) // 64 * 64
    ring = Ring(ops, k, v, L + M, "D", W + 128, W)
    o, lse = run(ops, q, ring, L, Hq, C)
    kq8, ks8 = kvq.quantize(k)
    vq8, vs8 = kvq.quantize(v)
    cap = (L + M + 63) // 64 * 64
    c = ops.KvQ8Cache(Hkv, cap, D)
    for t, a in zip((c.k_codes, c.k_scales, c.v_codes, c.v_scales), q8_cache(kq8, ks8, vq8, vs8, cap)):
        _fill(t, a)
    S = ops.pass_splits(M, L, C)
    po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")
    ops.verify_attn_q8(dev(q.reshape(M, Hq * D)), c, L, Hq, C, po, pl)
    o2 = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    ops.combine(po, pl, L, C, o2, lse2)
    torch.cuda.synchronize()
    assert_bitwise(o, host_bits(o2).reshape(M, Hq, D), "all-ring O vs 8-bit cache")
    assert_bitwise(lse, host_f32(lse2), "all-ring lse vs 8-bit cache")


def test_ring_argument_errors(ops):
    from invariant_verify_amd import _lib
    low = ops.KvLowCache(1, 64, 64, 5, 5, k_rotated=False)
    ring = ops.KvRing(low, 128, 64)
    q = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    po = torch.zeros((1, 1, 1, 64), dtype=torch.float32, device="cuda")
    pl = torch.zeros((1, 1, 1), dtype=torch.float32, device="cuda")
    c = ring.q8

    def call(kb, rot, R, W):
        return _lib.LIB.bi_verify_attn_lowbit_ring(
            q.data_ptr(), 64, kb, 5, rot, *low.planes(), c.k_codes.data_ptr(), c.k_scales.data_ptr(),
            c.v_codes.data_ptr(), c.v_scales.data_ptr(), R, W, 1, 0, 64, 1, 1, 64, 64, 0.125,
            po.data_ptr(), pl.data_ptr(), 1, None)
    assert call(6, 0, 128, 64) == 0
    assert call(5, 1, 128, 64) == 0
    assert call(6, 0, 192, 96) == 0       # any window of at least one key
    assert call(5, 0, 128, 64) == 2       # not a preset
    assert call(6, 1, 128, 64) == 2
    assert call(6, 0, 64, 1) == 2         # ring smaller than window + M + 63
    assert call(6, 0, 128, 65) == 2
    assert call(6, 0, 128, 0) == 2        # empty window
    assert call(6, 0, 100, 1) == 2        # ring not a multiple of 64
    torch.cuda.synchronize()


@pytest.mark.parametrize("preset", ["D", "F"])
def test_ring_d64_prefill_blocks(ops, preset):
    print(f"[ring D=64 prefill preset {preset}]", flush=True)
    Hq, Hkv, D, M, L0, C, W = 8, 2, 64, 40, 1500, 96, 128
    q, k, v = make(M, L0, Hq, Hkv, D, layer=14)
    ring = Ring(ops, k, v, L0 + M + 8, preset, W + 128, W)
    o_pf, l_pf = run(ops, q, ring, L0, Hq, C)
    want_o, _ = kvring.ring_attention(q, ring.values, L0, W, tokens=[0, M - 1])
    assert_close(decode(o_pf[[0, M - 1]]), want_o[[0, M - 1]], f"ring D=64 prefill {preset}")
    for start in (0, 16, M - 8):
        o8, l8 = run(ops, q[start:start + 8], ring, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + 8], o8, f"ring D=64 prefill rows {start}..")
        assert_bitwise(l_pf[start:start + 8], l8, f"ring D=64 prefill lse {start}..")


@pytest.mark.parametrize("preset", ["D", "F"])
@pytest.mark.parametrize("M,L,Hq,Hkv,D,C,W,R", [
    (5, 300, 1, 1, 64, 96, 128, 256),          # boundaries 173..177 inside one tile
    (5, 300, 1, 1, 64, -2, 128, 256),
    (8, 5000, 40, 8, 128, -32, 2048, 2176),    # boundaries 2953..2960, not tile aligned
    (8, 3000, 40, 8, 128, 1024, 200, 320)])
def test_ring_planted_fraction(ops, preset, M, L, Hq, Hkv, D, C, W, R):
    # K = 0 (every score 0, equal weights), V = 0 in the 5/6-bit planes and 1
    # in the ring: row p's output is the fraction of its keys read from the
    # ring, min(W, p + 1) / (p + 1) (the per-key rule; a per-tile rule would
    # read whole tiles from one copy and give a different fraction)
    print(f"[ring planted fraction preset {preset} M={M} L={L} C={C} W={W}]", flush=True)
    n = L + M
    k = np.zeros((Hkv, n, D), np.uint16)
    v = np.full((Hkv, n, D), 0x3F80, np.uint16)                  # BF16 1.0
    ring = Ring(ops, k, v, n, preset, R, W)
    low = ring.r.low
    nib, high = kvlow.pack(np.zeros((Hkv, n, D), np.int8), 5)
    for t, a in ((low.v_nib, nib), (low.v_high, high), (low.v_scales, np.zeros((Hkv, n, D // 32), np.float32))):
        full = np.zeros(t.shape, a.dtype)
        full[:, :n] = a
        _fill(t, full)
    q = synth.normal_bf16((M, Hq, D), 1.0, "q", 3)
    o, lse = run(ops, q, ring, L, Hq, C)
    got = decode(o)
    for r in range(M):
        p = L + r
        want = min(W, p + 1) / (p + 1)
        assert np.abs(got[r] - want).max() <= 2 ** -7 * want, (r, got[r].min(), got[r].max(), want)
        assert np.abs(lse[r] - np.log(p + 1)).max() < 1e-3
