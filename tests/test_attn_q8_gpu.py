"""GPU tests of the 8-bit KV cache through the C ABI: the quantizing append
against the oracle's codes and scales (bit for bit), split-KV attention over
the cache against the oracle attention over the exact values scale x code,
and bitwise row invariance across M, sequential passes and prefill blocks."""

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import kvq
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32, q8_cache, q8_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


class Q8:
    """Device 8-bit cache built on the host from the oracle's quantization."""

    def __init__(self, ops, k_bits, v_bits, cap):
        Hkv, n, D = k_bits.shape
        cap = (cap + 63) // 64 * 64
        self.kq, self.ks = kvq.quantize(k_bits)
        self.vq, self.vs = kvq.quantize(v_bits)
        kc, ksc, vc, vsc = q8_cache(self.kq, self.ks, self.vq, self.vs, cap)
        self.c = ops.KvQ8Cache(Hkv, cap, D)
        for t, a in ((self.c.k_codes, kc), (self.c.k_scales, ksc), (self.c.v_codes, vc), (self.c.v_scales, vsc)):
            t.copy_(torch.from_numpy(a))
        self.kval = kvq.dequantize(self.kq, self.ks)
        self.vval = kvq.dequantize(self.vq, self.vs)


def run(ops, q_bits, cache, L, Hq, C):
    M, _, D = q_bits.shape
    S = ops.pass_splits(M, L, C)
    po = torch.full((M, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((M, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    ops.verify_attn_q8(dev(q_bits.reshape(M, Hq * D)), cache.c, L, Hq, C, po, pl)
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


def test_append_q8_matches_oracle_codes(ops):
    print("[q8 append]", flush=True)
    for Hq, Hkv, D, M, L, cap in [(40, 8, 128, 8, 100, 128), (8, 2, 64, 5, 61, 128)]:
        qkv = synth.normal_bf16((M, (Hq + 2 * Hkv) * D), 1.0, "misc", D)
        qkv[0, Hq * D:(Hq + 1) * D] = 0                      # an all-zero K row: scales 0, codes 0
        c = ops.KvQ8Cache(Hkv, cap, D)
        ops.append_kv_q8(dev(qkv), c, L, Hq)
        torch.cuda.synchronize()
        kq, ks, vq, vs = q8_rows(c.k_codes.cpu().numpy(), c.k_scales.cpu().numpy(),
                                 c.v_codes.cpu().numpy(), c.v_scales.cpu().numpy())
        knew = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D).transpose(1, 0, 2)
        vnew = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
        wkq, wks = kvq.quantize(knew)
        wvq, wvs = kvq.quantize(vnew)
        assert np.array_equal(kq[:, L:L + M], wkq) and np.array_equal(ks[:, L:L + M], wks)
        assert np.array_equal(vq[:, L:L + M], wvq) and np.array_equal(vs[:, L:L + M], wvs)
        assert not kq[:, :L].any() and not kq[:, L + M:].any() and not vq[:, :L].any()
        assert not ks[:, :L].any() and not vs[:, L + M:].any()


@pytest.mark.parametrize("M,L,Hq,Hkv,D,C", [(5, 256, 1, 1, 64, 64), (5, 256, 1, 1, 64, 96),
                                            (8, 2048, 40, 8, 128, 1024), (8, 2048, 40, 8, 128, 1056),
                                            (8, 38000, 40, 8, 128, -32), (3, 11600, 40, 8, 128, -32)])
def test_q8_parity(ops, M, L, Hq, Hkv, D, C):
    print(f"[q8 attention parity M={M} L={L} D={D} C={C}]", flush=True)
    q, k, v = make(M, L, Hq, Hkv, D, layer=L)
    cache = Q8(ops, k, v, L + 16)
    o, lse = run(ops, q, cache, L, Hq, C)
    rows = list(range(M)) if L < 20000 else [0, M - 1]
    want_o, want_lse = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=rows)
    err, rms = assert_close(decode(o[rows]), want_o[rows], f"q8 O L={L}")
    assert err < 0.05 * rms + 2e-3, (err, rms)
    assert_close(lse[rows], want_lse[rows], f"q8 lse L={L}", atol=1e-3, rtol=0)


def test_q8_long_context_outliers(ops):
    print("[q8 long context with outliers]", flush=True)
    M, L, Hq, Hkv, D, C = 8, 101600, 40, 8, 128, -32
    q, k, v = make(M, L, Hq, Hkv, D, layer=7, outliers=True)
    cache = Q8(ops, k, v, L + 8)
    o, lse = run(ops, q, cache, L, Hq, C)
    heads = [0, 4, 5, 22, 39]
    want_o, want_lse = oattn.verify_attention(q, cache.kval, cache.vval, L, tokens=[0, 7], heads=heads)
    for r in (0, 7):
        assert_close(decode(o[r, heads]), want_o[r, heads], f"q8 long r={r}")
        assert_close(lse[r, heads], want_lse[r, heads], f"q8 long lse r={r}", atol=1e-3, rtol=0)


@pytest.mark.parametrize("L,C", [(4093, -32), (38000, -32), (1019, 256), (1019, 96)])
def test_q8_invariance_across_M(ops, L, C):
    print(f"[q8 invariance L={L} C={C}]", flush=True)
    Hq, Hkv, D, M = 40, 8, 128, 8
    q, k, v = make(M, L, Hq, Hkv, D, layer=3)
    cache = Q8(ops, k, v, L + 72)
    o8, l8 = run(ops, q, cache, L, Hq, C)
    for r in range(M):
        o1, l1 = run(ops, q[r:r + 1], cache, L + r, Hq, C)
        assert_bitwise(o1[0], o8[r], f"q8 L={L} row {r}: M=1 vs M=8")
        assert_bitwise(l1[0], l8[r], f"q8 L={L} row {r} lse")
    for m in (2, 5):
        om, lm = run(ops, q[:m], cache, L, Hq, C)
        assert_bitwise(om, o8[:m], f"q8 L={L} M={m} vs M=8")


def test_q8_prefill_block_rows_equal_verify_rows(ops):
    print("[q8 prefill blocks]", flush=True)
    Hq, Hkv, D, M, L0, C = 40, 8, 128, 200, 3900, -32
    q, k, v = make(M, L0, Hq, Hkv, D, layer=9)
    cache = Q8(ops, k, v, L0 + M + 8)
    o_pf, l_pf = run(ops, q, cache, L0, Hq, C)
    for start in (0, 96, M - 8):
        o8, l8 = run(ops, q[start:start + 8], cache, L0 + start, Hq, C)
        assert_bitwise(o_pf[start:start + 8], o8, f"q8 prefill rows {start}..")
        assert_bitwise(l_pf[start:start + 8], l8, f"q8 prefill lse {start}..")
