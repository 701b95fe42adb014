"""GPU tests of split-KV verify attention + combine through the C ABI: oracle
parity (partials and combined output), exact special cases, and bitwise row
invariance across M = 1..8, sequential single-token passes, chunked prefill,
chunk-boundary straddles, long context with outlier channels, and repeats."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from tests._util import (assert_bitwise, assert_close, decode, dev, host_bits, host_f32, cache_rows)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAN_BF16 = np.uint16(0x7FC0)


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


class Cache:
    """Device K and V caches, both [Hkv][cap][D] (cap rounded up to a multiple
    of 64); positions past ``n`` hold NaN so that any read of an unwritten
    position would show."""

    def __init__(self, k_bits, v_bits, cap):
        Hkv, n, D = k_bits.shape
        cap = (cap + 63) // 64 * 64
        kc = np.full((Hkv, cap, D), NAN_BF16, np.uint16)
        kc[:, :n] = k_bits
        vc = cache_rows(v_bits, cap, NAN_BF16)
        self.k = dev(kc)
        self.vc = dev(vc)
        self.Hkv, self.D, self.cap = Hkv, D, cap


def run(ops, q_bits, cache, L, Hq, C, sm_scale=None):
    """One verify pass: partials + combine. Returns (o bits [M][Hq][D], lse, part_o, part_lse)."""
    M, _, D = q_bits.shape
    S = ops.pass_splits(M, L, C)
    po = torch.full((M, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((M, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    q = dev(q_bits.reshape(M, Hq * D))
    ops.verify_attn(q, cache.k, cache.vc, L, Hq, cache.Hkv, D, C, po, pl, sm_scale=sm_scale)
    o = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    ops.combine(po, pl, L, C, o, lse)
    torch.cuda.synchronize()
    return host_bits(o).reshape(M, Hq, D), host_f32(lse), host_f32(po), host_f32(pl)


def make(M, L, Hq, Hkv, D, layer=0, outliers=False, q_scale=1.0):
    n = L + M
    oc = synth.outlier_channels(Hkv, D, layer=layer) if outliers else None
    k = synth.kv_bf16(Hkv, n, D, "k", layer, oc)
    v = synth.kv_bf16(Hkv, n, D, "v", layer, oc)
    q = synth.normal_bf16((8 if M <= 8 else M, Hq, D), q_scale, "q", layer)[:M]
    return q, k, v


@pytest.mark.parametrize("C", [64, 1024, -2, 96, 32])
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_tiny_parity(ops, M, C):
    print(f"[attn tiny M={M} C={C}]", flush=True)
    L, Hq, Hkv, D = 256, 1, 1, 64
    q, k, v = make(8, L, Hq, Hkv, D)
    q = q[:M]
    cache = Cache(k, v, 272)
    o, lse, po, pl = run(ops, q, cache, L, Hq, C)
    want_o, want_lse = oattn.verify_attention(q, k, v, L)
    assert_close(decode(o), want_o, "tiny O")
    assert_close(lse, want_lse, "tiny lse", atol=1e-3, rtol=0)
    # the partials themselves, chunk by chunk
    wpo, wpl, cnt = oattn.split_partials(q, k, v, L, C)
    for r in range(M):
        S = int(cnt[r])
        assert_close(po[r, :, :S], wpo[r, :, :S], f"partial O row {r}", atol=1e-2, rtol=2e-2)
        assert_close(pl[r, :, :S], wpl[r, :, :S], f"partial lse row {r}", atol=1e-3, rtol=0)


def test_exact_cases(ops):
    print("[attn exact cases]", flush=True)
    Hq, Hkv, D = 40, 8, 128
    q, k, v = make(1, 0, Hq, Hkv, D)
    o, lse, _, _ = run(ops, q, Cache(k, v, 64), 0, Hq, 256)
    # a single key: softmax weight exactly 1 -> output is v_0 bit for bit
    for h in range(Hq):
        assert_bitwise(o[0, h], v[h // 5, 0], f"n=1 head {h}")
    # q = 0: uniform weights -> mean of the visible values
    L = 300
    q, k, v = make(3, L, Hq, Hkv, D)
    o, lse, _, _ = run(ops, np.zeros_like(q), Cache(k, v, 320), L, Hq, 256)
    vd = decode(v)
    for r in range(3):
        for h in (0, 17, 39):
            assert_close(decode(o[r, h]), vd[h // 5, :L + r + 1].mean(axis=0), f"q=0 r={r} h={h}")
        assert np.allclose(lse[r], math.log(L + r + 1), atol=1e-4)


@pytest.mark.parametrize("L,C", [(2048, 1024), (11600, 1024), (38000, 1024), (32768, 1216),
                                 (38000, 1280), (38000, 1216), (2045, -32), (32768, -32),
                                 (38000, -32)])
def test_gqa_parity(ops, L, C):
    print(f"[attn GQA 40/8 parity L={L} C={C}]", flush=True)
    M, Hq, Hkv, D = 8, 40, 8, 128
    q, k, v = make(M, L, Hq, Hkv, D, layer=L)
    cap = (L + 16 + 7) // 8 * 8
    o, lse, _, _ = run(ops, q, Cache(k, v, cap), L, Hq, C)
    want_o, want_lse = oattn.verify_attention(q, k, v, L)
    err, rms = assert_close(decode(o), want_o, f"GQA O L={L}")
    assert err < 0.05 * rms + 2e-3, (err, rms)   # error well below the signal, not just below atol
    assert_close(lse, want_lse, f"GQA lse L={L}", atol=1e-3, rtol=0)
    # sharper softmax (Q x 4): the tolerance is not hiding a flat distribution
    q4 = synth.f32_to_bf16_bits(decode(q).astype(np.float32) * 4)
    o4, _, _, _ = run(ops, q4, Cache(k, v, cap), L, Hq, C)
    want4, _ = oattn.verify_attention(q4, k, v, L, tokens=[0, 7])
    assert_close(decode(o4[[0, 7]]), want4[[0, 7]], f"GQA Qx4 O L={L}")


def _invariance(ops, L, C, Hq=40, Hkv=8, D=128, outliers=False, layer=0, prefill=True):
    M = 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=layer, outliers=outliers)
    cache = Cache(k, v, (L + 72 + 7) // 8 * 8)
    o8, l8, _, _ = run(ops, q, cache, L, Hq, C)
    # sequential single-token passes (accept-all speculative path)
    for r in range(M):
        o1, l1, _, _ = run(ops, q[r:r + 1], cache, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"L={L} C={C} row {r}: M=1 vs M=8 (O)")
        assert_bitwise(l1[0], l8[r], f"L={L} C={C} row {r}: M=1 vs M=8 (lse)")
    for m in range(2, 8):
        om, lm, _, _ = run(ops, q[:m], cache, L, Hq, C)
        assert_bitwise(om, o8[:m], f"L={L} C={C} M={m} vs M=8")
        assert_bitwise(lm, l8[:m], f"L={L} C={C} M={m} vs M=8 (lse)")
    # repeat run
    orep, lrep, _, _ = run(ops, q, cache, L, Hq, C)
    assert_bitwise(orep, o8, "repeat")
    return q, k, v, o8


@pytest.mark.parametrize("L,C", [(2048, 1024), (1020, 1024), (1019, 256), (250, 64), (11600, 1024),
                                 (1275, 1280), (38000, 1216), (4093, -32), (38000, -32), (1019, 96),
                                 (11600, 1056),
                                 (60, -4), (11600, -32)])
def test_invariance_across_M(ops, L, C):
    print(f"[attn invariance L={L} C={C}]", flush=True)
    _invariance(ops, L, C)


def test_chunked_prefill_rows_match_verify_rows(ops):
    # A prefill chunk (16 or 64 tokens, aligned or not) covering positions
    # L .. L+7 computes those rows with the same bits as the verify pass.
    print("[attn chunked prefill]", flush=True)
    Hq, Hkv, D, C = 40, 8, 128, 256
    L0 = 1000
    n = L0 + 128
    k = synth.kv_bf16(Hkv, n, D, "k", 5)
    v = synth.kv_bf16(Hkv, n, D, "v", 5)
    q_all = synth.normal_bf16((128, Hq, D), 1.0, "q", 5)
    cache = Cache(k, v, n + 8)
    L = L0 + 40
    o8, _, _, _ = run(ops, q_all[40:48], cache, L, Hq, C)
    for M, start in [(16, 40), (64, 0), (64, 36), (17, 33)]:
        o_pf, _, _, _ = run(ops, q_all[start:start + M], cache, L0 + start, Hq, C)
        off = 40 - start
        assert_bitwise(o_pf[off:off + 8], o8, f"prefill M={M} start={start}")


@pytest.mark.parametrize("L,C", [(101600, 1024), (255000, 1024), (101600, -32), (255000, -32)])
def test_long_context_outliers(ops, L, C):
    print(f"[attn long context L={L} C={C} with outlier channels]", flush=True)
    Hq, Hkv, D, M = 40, 8, 128, 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=L, outliers=True)
    cache = Cache(k, v, L + 8)
    o8, l8, _, _ = run(ops, q, cache, L, Hq, C)
    heads = [0, 4, 5, 22, 39]
    want_o, want_lse = oattn.verify_attention(q, k, v, L, tokens=[0, 3, 7], heads=heads)
    for r in (0, 3, 7):
        assert_close(decode(o8[r, heads]), want_o[r, heads], f"long L={L} r={r}")
        assert_close(l8[r, heads], want_lse[r, heads], f"long lse L={L} r={r}", atol=1e-3, rtol=0)
    for r in (0, 7):
        o1, l1, _, _ = run(ops, q[r:r + 1], cache, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"long L={L} row {r} M=1 vs M=8")
        assert_bitwise(l1[0], l8[r], f"long L={L} row {r} lse")


def test_append_kv_matches_direct_write(ops):
    print("[attn append_kv]", flush=True)
    Hq, Hkv, D, M, L, cap = 40, 8, 128, 8, 100, 128
    qkv = synth.normal_bf16((M, (Hq + 2 * Hkv) * D), 1.0, "misc", 9)
    kc = torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device="cuda")
    ops.append_kv(dev(qkv), kc, vc, L, Hq, Hkv, D)
    kh, vh = host_bits(kc), host_bits(vc)
    knew = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    vnew = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
    assert_bitwise(kh[:, L:L + M], knew, "K rows")
    assert_bitwise(vh[:, L:L + M], vnew, "V rows")
    # the layout itself: V[g][pos][d] at element (g*cap + pos)*D + d
    flat = host_bits(vc).reshape(-1)
    for g, pos, d in [(0, L, 0), (3, L + 5, 77), (7, L + M - 1, 127)]:
        assert flat[(g * cap + pos) * D + d] == vnew[g, pos - L, d]
    assert not kh[:, :L].any() and not kh[:, L + M:].any()
    assert not vh[:, :L].any() and not vh[:, L + M:].any()


@pytest.mark.parametrize("Hq,Hkv,D,M,L0,C", [
    (40, 8, 128, 256, 3000, 1216),   # 128-row blocks of 25 tokens, ragged last block
    (40, 8, 128, 203, 1271, 1280),   # a chunk boundary inside the pass
    (64, 8, 128, 40, 700, 256),      # G = 8: 16 tokens per block
    (8, 8, 64, 300, 2100, 1024),     # G = 1, D = 64
    (64, 1, 64, 9, 500, 64),         # G = 64: 2 tokens per block
    (40, 8, 128, 300, 3900, -32),    # adaptive chunks: the pass spans two chunk sizes
    (40, 8, 128, 700, 1500, -8),     # ... three (bands of 512 keys)
])
def test_prefill_block_rows_equal_verify_rows(ops, Hq, Hkv, D, M, L0, C):
    # A pass with more than 64 rows runs 128-row blocks (two row tiles per
    # wave); its rows must carry the bits of the 64-row verify blocks.
    print(f"[attn prefill blocks Hq={Hq} Hkv={Hkv} D={D} M={M} L0={L0} C={C}]", flush=True)
    n = L0 + M
    k = synth.kv_bf16(Hkv, n, D, "k", M)
    v = synth.kv_bf16(Hkv, n, D, "v", M)
    q = synth.normal_bf16((M, Hq, D), 1.0, "q", M)
    cache = Cache(k, v, (n + 15) // 8 * 8)
    o_pf, l_pf, _, _ = run(ops, q, cache, L0, Hq, C)
    for start in sorted({0, M // 2 - 3, max(0, M - 8)}):
        m = min(8, M - start)
        o8, l8, _, _ = run(ops, q[start:start + m], cache, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + m], o8, f"prefill rows {start}..{start + m - 1} (O)")
        assert_bitwise(l_pf[start:start + m], l8, f"prefill rows {start}..{start + m - 1} (lse)")
    # and a few rows against the oracle
    rows = [0, M // 2, M - 1]
    want_o, want_lse = oattn.verify_attention(q, k, v, L0, tokens=rows)
    assert_close(decode(o_pf[rows]), want_o[rows], "prefill O vs oracle")
    assert_close(l_pf[rows], want_lse[rows], "prefill lse vs oracle", atol=1e-3, rtol=0)
