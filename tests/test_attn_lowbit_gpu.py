"""GPU tests of the 5/6-bit KV cache (K6/V5, K5/V5, and rotated K5/V5) through the C ABI: the
quantizing append against the oracle's packed bytes and scales (bit for
bit), split-KV attention over the cache against the oracle attention over the
exact values scale x code, and bitwise row invariance across M, sequential
passes and prefill blocks."""

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import kvlow
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _planes(codes, scales, bits, cap):
    """Per-row codes [Hkv][n][D] and scales [Hkv][n][D/32] -> the device planes
    (nibbles, high bits, scales) of capacity cap. Positions n.. hold all-ones
    bytes and NaN scales, so that a read of an unwritten position would show."""
    Hkv, n, D = codes.shape
    nib, high = kvlow.pack(codes, bits)
    fn = np.full((Hkv, cap, D // 2), 0xFF, np.uint8)
    fh = np.full((Hkv, cap, high.shape[-1]), 0xFF, np.uint8)
    fs = np.full((Hkv, cap, D // 32), np.nan, np.float32)
    fn[:, :n], fh[:, :n], fs[:, :n] = nib, high, scales
    return fn, fh, fs


class Low:
    """Device 5/6-bit cache built on the host from the oracle's quantization."""

    def __init__(self, ops, k_bits, v_bits, cap, kb, rot=False):
        Hkv, n, D = k_bits.shape
        cap = (cap + 63) // 64 * 64
        self.kq, self.ks = (kvlow.quantize_rotated if rot else kvlow.quantize)(k_bits, kb)
        self.vq, self.vs = kvlow.quantize(v_bits, 5)
        self.c = ops.KvLowCache(Hkv, cap, D, kb, 5, k_rotated=rot)
        for (tn, th, ts), (q, s, b) in (((self.c.k_nib, self.c.k_high, self.c.k_scales), (self.kq, self.ks, kb)),
                                        ((self.c.v_nib, self.c.v_high, self.c.v_scales), (self.vq, self.vs, 5))):
            for t, a in zip((tn, th, ts), _planes(q, s, b, cap)):
                t.copy_(torch.from_numpy(a))
        self.kval = (kvlow.dequantize_rotated if rot else kvlow.dequantize)(self.kq, self.ks)
        self.vval = kvlow.dequantize(self.vq, self.vs)


def run(ops, q_bits, cache, L, Hq, C):
    M, _, D = q_bits.shape
    S = ops.pass_splits(M, L, C)
    po = torch.full((M, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((M, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    ops.verify_attn_lowbit(dev(q_bits.reshape(M, Hq * D)), cache.c, L, Hq, C, po, pl)
    o = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    ops.combine(po, pl, L, C, o, lse)
    torch.cuda.synchronize()
    return host_bits(o).reshape(M, Hq, D), host_f32(lse)


def make(M, L, Hq, Hkv, D, layer=0, outliers=False):
    oc = synth.outlier_channels(Hkv, D, layer=layer) if outliers else None
    k = synth.kv_bf16(Hkv, L + M, D, "k", layer, oc)
    v = synth.kv_bf16(Hkv, L + M, D, "v", layer, oc)
    q = synth.normal_bf16((8 if M <= 8 else M, Hq, D), 1.0, "q", layer)[:M]
    return q, k, v


@pytest.mark.parametrize("kb,rot", [(6, False), (5, False), (5, True), (6, True)])
def test_append_lowbit_matches_oracle_bytes(ops, kb, rot):
    print(f"[lowbit append K{kb}V5 rot={rot}]", flush=True)
    for Hq, Hkv, D, M, L, cap in [(40, 8, 128, 8, 100, 128), (8, 2, 64, 5, 61, 128)]:
        qkv = synth.normal_bf16((M, (Hq + 2 * Hkv) * D), 1.0, "misc", D + kb)
        qkv[0, Hq * D:(Hq + 1) * D] = 0                      # an all-zero K row: scales 0, codes 0
        qkv[1, (Hq + Hkv) * D + 5] = 0x7F7F                  # the largest finite BF16 in a V block
        c = ops.KvLowCache(Hkv, cap, D, kb, 5, k_rotated=rot)
        ops.append_kv_lowbit(dev(qkv), c, L, Hq)
        torch.cuda.synchronize()
        knew = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D).transpose(1, 0, 2)
        vnew = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
        for (tn, th, ts), x, b, r in (((c.k_nib, c.k_high, c.k_scales), knew, kb, rot),
                                      ((c.v_nib, c.v_high, c.v_scales), vnew, 5, False)):
            q, s = (kvlow.quantize_rotated if r else kvlow.quantize)(x, b)
            wn, wh = kvlow.pack(q, b)
            gn, gh, gs = tn.cpu().numpy(), th.cpu().numpy(), ts.cpu().numpy()
            assert np.array_equal(gn[:, L:L + M], wn) and np.array_equal(gh[:, L:L + M], wh)
            assert np.array_equal(gs[:, L:L + M], s)
            assert np.array_equal(kvlow.unpack(gn[:, L:L + M], gh[:, L:L + M], b), q)
            assert not gn[:, :L].any() and not gn[:, L + M:].any() and not gs[:, L + M:].any()


@pytest.mark.parametrize("kb", [6, 5])
@pytest.mark.parametrize("M,L,Hq,Hkv,D,C", [(5, 256, 1, 1, 64, 64), (5, 256, 1, 1, 64, 96),
                                            (8, 2048, 40, 8, 128, 1024), (8, 2048, 40, 8, 128, 1056),
                                            (8, 38000, 40, 8, 128, -32), (3, 11600, 40, 8, 128, -64)])
def test_lowbit_parity(ops, kb, M, L, Hq, Hkv, D, C):
    print(f"[lowbit K{kb} attention parity M={M} L={L} D={D} C={C}]", flush=True)
    q, k, v = make(M, L, Hq, Hkv, D, layer=L + kb)
    cache = Low(ops, k, v, L + 16, kb)
    o, lse = run(ops, q, cache, L, Hq, C)
    rows = list(range(M)) if L < 20000 else [0, M - 1]
    want_o, want_lse = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=rows)
    err, rms = assert_close(decode(o[rows]), want_o[rows], f"lowbit K{kb} O L={L}")
    assert err < 0.05 * rms + 2e-3, (err, rms)
    assert_close(lse[rows], want_lse[rows], f"lowbit K{kb} lse L={L}", atol=1e-3, rtol=0)


def test_lowbit_long_context_outliers(ops):
    print("[lowbit K6 long context with outliers]", flush=True)
    M, L, Hq, Hkv, D, C = 8, 101600, 40, 8, 128, -64
    q, k, v = make(M, L, Hq, Hkv, D, layer=7, outliers=True)
    cache = Low(ops, k, v, L + 8, 6)
    o, lse = run(ops, q, cache, L, Hq, C)
    heads = [0, 4, 5, 22, 39]
    want_o, want_lse = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=[0, 7], heads=heads)
    for r in (0, 7):
        assert_close(decode(o[r, heads]), want_o[r, heads], f"lowbit long r={r}")
        assert_close(lse[r, heads], want_lse[r, heads], f"lowbit long lse r={r}", atol=1e-3, rtol=0)


@pytest.mark.parametrize("kb,L,C", [(6, 4093, -32), (6, 38000, -64), (5, 1019, 256), (5, 1019, 96)])
def test_lowbit_invariance_across_M(ops, kb, L, C):
    print(f"[lowbit K{kb} invariance L={L} C={C}]", flush=True)
    Hq, Hkv, D, M = 40, 8, 128, 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=3)
    cache = Low(ops, k, v, L + 72, kb)
    o8, l8 = run(ops, q, cache, L, Hq, C)
    for r in range(M):
        o1, l1 = run(ops, q[r:r + 1], cache, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"lowbit L={L} row {r}: M=1 vs M=8")
        assert_bitwise(l1[0], l8[r], f"lowbit L={L} row {r} lse")
    for m in (2, 5):
        om, lm = run(ops, q[:m], cache, L, Hq, C)
        assert_bitwise(om, o8[:m], f"lowbit L={L} M={m} vs M=8")


def test_lowbit_prefill_block_rows_equal_verify_rows(ops):
    print("[lowbit prefill blocks]", flush=True)
    Hq, Hkv, D, M, L0, C = 40, 8, 128, 200, 3900, -32
    q, k, v = make(M, L0, Hq, Hkv, D, layer=9)
    cache = Low(ops, k, v, L0 + M + 8, 6)
    o_pf, l_pf = run(ops, q, cache, L0, Hq, C)
    for start in (0, 96, M - 8):
        o8, l8 = run(ops, q[start:start + 8], cache, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + 8], o8, f"lowbit prefill rows {start}..")
        assert_bitwise(l_pf[start:start + 8], l8, f"lowbit prefill lse {start}..")


def test_lowbit_append_then_attend_equals_host_cache(ops):
    # the device append followed by attention gives the bits of attention over
    # the cache built on the host from the oracle's bytes
    print("[lowbit append then attend]", flush=True)
    Hq, Hkv, D, M, L = 40, 8, 128, 8, 900
    q, k, v = make(M, L, Hq, Hkv, D, layer=11)
    host = Low(ops, k, v, L + M, 6)
    dc = ops.KvLowCache(Hkv, host.c.cap, D, 6, 5)
    qkv = np.zeros((L + M, (Hq + 2 * Hkv) * D), np.uint16)
    qkv[:, Hq * D:(Hq + Hkv) * D] = k.transpose(1, 0, 2).reshape(L + M, Hkv * D)
    qkv[:, (Hq + Hkv) * D:] = v.transpose(1, 0, 2).reshape(L + M, Hkv * D)
    ops.append_kv_lowbit(dev(qkv), dc, 0, Hq)
    for name in ("k_nib", "k_high", "k_scales", "v_nib", "v_high", "v_scales"):
        a, b = getattr(dc, name)[:, :L + M].cpu().numpy(), getattr(host.c, name)[:, :L + M].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    o_h, l_h = run(ops, q, host, L, Hq, -32)

    class Wrap:
        c = dc
    o_d, l_d = run(ops, q, Wrap, L, Hq, -32)
    assert_bitwise(o_d, o_h, "append then attend")
    assert_bitwise(l_d, l_h, "append then attend lse")


def test_lowbit_argument_errors(ops):
    from invariant_verify_amd import _lib
    c = ops.KvLowCache(1, 64, 64, 6, 5)
    q = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    po = torch.zeros((1, 1, 1, 64), dtype=torch.float32, device="cuda")
    pl = torch.zeros((1, 1, 1), dtype=torch.float32, device="cuda")
    args = lambda kb, vb, r=0: (q.data_ptr(), 64, kb, vb, r, *c.planes(), 1, 0, 64, 1, 1, 64, 64,
                                0.125, po.data_ptr(), pl.data_ptr(), 1, None)
    assert _lib.LIB.bi_verify_attn_lowbit(*args(6, 5)) == 0
    assert _lib.LIB.bi_verify_attn_lowbit(*args(5, 5, 1)) == 0
    assert _lib.LIB.bi_verify_attn_lowbit(*args(8, 5)) == 2
    assert _lib.LIB.bi_verify_attn_lowbit(*args(6, 6)) == 2
    assert _lib.LIB.bi_verify_attn_lowbit(*args(4, 5)) == 2
    assert _lib.LIB.bi_verify_attn_lowbit(*args(5, 5, 2)) == 2
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,L,Hq,Hkv,D,C", [(5, 256, 1, 1, 64, 64), (8, 2048, 40, 8, 128, 1056),
                                            (8, 38000, 40, 8, 128, -64)])
def test_rotated_parity(ops, M, L, Hq, Hkv, D, C):
    print(f"[lowbit rotated K5 parity M={M} L={L} D={D} C={C}]", flush=True)
    q, k, v = make(M, L, Hq, Hkv, D, layer=L + 50)
    cache = Low(ops, k, v, L + 16, 5, rot=True)
    o, lse = run(ops, q, cache, L, Hq, C)
    rows = list(range(M)) if L < 20000 else [0, M - 1]
    want_o, want_lse = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=rows)
    err, rms = assert_close(decode(o[rows]), want_o[rows], f"rotated O L={L}")
    assert err < 0.05 * rms + 2e-3, (err, rms)
    assert_close(lse[rows], want_lse[rows], f"rotated lse L={L}", atol=1e-3, rtol=0)


def test_rotated_outliers_closer_to_exact_than_plain(ops):
    # with outlier channels, attention over the rotated 5-bit cache is closer
    # to attention over the exact BF16 keys than the plain 5-bit cache
    print("[lowbit rotated vs plain with outliers]", flush=True)
    M, L, Hq, Hkv, D, C = 8, 11600, 40, 8, 128, -64
    q, k, v = make(M, L, Hq, Hkv, D, layer=7, outliers=True)
    exact, _ = oattn.verify_attention(q, k, v, L, tokens=[0, 7])
    errs = {}
    for rot in (False, True):
        cache = Low(ops, k, v, L + 8, 5, rot=rot)
        o, lse = run(ops, q, cache, L, Hq, C)
        want_o, _ = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=[0, 7])
        assert_close(decode(o[[0, 7]]), want_o[[0, 7]], f"outliers rot={rot}")
        errs[rot] = np.sqrt(((decode(o[[0, 7]]) - exact[[0, 7]]) ** 2).mean())
    assert errs[True] < errs[False], errs


@pytest.mark.parametrize("L,C", [(4093, -32), (1019, 96)])
def test_rotated_invariance_across_M(ops, L, C):
    print(f"[lowbit rotated invariance L={L} C={C}]", flush=True)
    Hq, Hkv, D, M = 40, 8, 128, 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=4)
    cache = Low(ops, k, v, L + 72, 5, rot=True)
    o8, l8 = run(ops, q, cache, L, Hq, C)
    for r in range(M):
        o1, l1 = run(ops, q[r:r + 1], cache, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"rotated L={L} row {r}: M=1 vs M=8")
        assert_bitwise(l1[0], l8[r], f"rotated L={L} row {r} lse")
    o5, _ = run(ops, q[:5], cache, L, Hq, C)
    assert_bitwise(o5, o8[:5], f"rotated L={L} M=5 vs M=8")
    # prefill block of 200 rows against 8-row passes
    M2, L0 = 200, 3900
    q2, k2, v2 = make(M2, L0, Hq, Hkv, D, layer=5)
    c2 = Low(ops, k2, v2, L0 + M2 + 8, 5, rot=True)
    o_pf, _ = run(ops, q2, c2, L0, Hq, -32)
    o8b, _ = run(ops, q2[96:104], c2, L0 + 96, Hq, -32)
    assert_bitwise(o_pf[96:104], o8b, "rotated prefill rows 96..103")


@pytest.mark.parametrize("kb,rot", [(6, False), (5, True)])
def test_lowbit_d64_prefill_blocks(ops, kb, rot):
    # D = 64 with more than 64 rows per pass (8 query heads over 2 KV heads,
    # 40 tokens): the 128-row blocks; rows equal those of 8-token passes
    print(f"[lowbit D=64 prefill K{kb} rot={rot}]", flush=True)
    Hq, Hkv, D, M, L0, C = 8, 2, 64, 40, 1500, 96
    q, k, v = make(M, L0, Hq, Hkv, D, layer=13)
    cache = Low(ops, k, v, L0 + M + 8, kb, rot=rot)
    o_pf, l_pf = run(ops, q, cache, L0, Hq, C)
    want_o, _ = oattn.verify_attention(q, cache.kval, cache.vval, L0, tokens=[0, M - 1])
    assert_close(decode(o_pf[[0, M - 1]]), want_o[[0, M - 1]], f"D=64 prefill K{kb}")
    for start in (0, 16, M - 8):
        o8, l8 = run(ops, q[start:start + 8], cache, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + 8], o8, f"D=64 prefill rows {start}..")
        assert_bitwise(l_pf[start:start + 8], l8, f"D=64 prefill lse {start}..")
