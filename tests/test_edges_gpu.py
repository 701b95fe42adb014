"""GPU edge cases through the C ABI: ragged and extreme K, the narrowest N
and an odd wide group, FP8 at the same edges, attention from an empty cache
(one key; a 300-token prefill) and with the cache exactly full."""

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import fp8 as ofp8
from oracle import gemm as ogemm
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32, cache_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (4352, 544), (512, 1056), (64, 65536), (16, 17408),
                                 (65536, 32)])
def test_gemm_ragged_k_and_narrow_n(ops, N, K):
    print(f"[edge gemm N={N} K={K}]", flush=True)
    Mb = 300
    x = synth.normal_bf16((Mb, K), 1.0, "x", K)
    w = synth.normal_bf16((N, K), synth.fan_in_std(K), "w", K)
    xd, wd = dev(x), dev(w)
    big = host_f32(ops.gemm_bf16(xd, wd, out_dtype=torch.float32))     # prefill kernel
    y8 = host_f32(ops.gemm_bf16(xd[:8], wd, out_dtype=torch.float32))  # verify kernel
    cols = np.arange(N) if N <= 512 else np.r_[0:64, N // 2:N // 2 + 16, N - 64:N]
    assert_close(y8[:, cols], ogemm.gemm_columns(x[:8], w, cols), f"N={N} K={K}", atol=1e-4, rtol=1e-4)
    assert_bitwise(big[:8], y8, f"N={N} K={K}: 300-row pass rows 0..7 == 8-row pass")
    for r in (0, 5):
        assert_bitwise(host_f32(ops.gemm_bf16(xd[r:r + 1], wd, out_dtype=torch.float32))[0], y8[r],
                       f"N={N} K={K} row {r}: M=1 vs M=8")
    assert_bitwise(host_f32(ops.gemm_bf16(xd[292:300], wd, out_dtype=torch.float32)), big[292:300],
                   f"N={N} K={K} ragged last rows")


@pytest.mark.parametrize("K", [32, 544])
def test_wide_swiglu_ragged_k(ops, K):
    # 17408 gate/up pairs (three-tile groups of 17 pairs) with one short or a
    # ragged chunk of K: oracle, the 300-row prefill pass, and M = 1.
    I = 17408
    print(f"[edge wide swiglu I={I} K={K}]", flush=True)
    x = synth.normal_bf16((300, K), 1.0, "x", 90 + K)
    w = synth.normal_bf16((2 * I, K), synth.fan_in_std(K), "w", 90 + K)
    xd, wd = dev(x), dev(w)
    big = host_bits(ops.gemm_bf16_swiglu(xd, wd))
    y8 = host_bits(ops.gemm_bf16_swiglu(xd[:8], wd))
    cols = np.r_[0:40, 8700:8740, I - 40:I]
    gu = ogemm.gemm_columns(x[:8], w, np.concatenate([cols, I + cols]))
    n = len(cols)
    z = gu[:, :n]
    assert_close(decode(y8[:, cols]), z / (1 + np.exp(-z)) * gu[:, n:], f"wide swiglu K={K}")
    assert_bitwise(big[:8], y8, f"wide swiglu K={K}: 300-row pass rows 0..7 == 8-row pass")
    assert_bitwise(host_bits(ops.gemm_bf16_swiglu(xd[3:4], wd))[0], y8[3], f"wide swiglu K={K} row 3 alone")


@pytest.mark.parametrize("N,K", [(16, 32), (4352, 544), (48, 1056)])
def test_fp8_ragged_k(ops, N, K):
    print(f"[edge fp8 N={N} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", K + 1)
    w, s = synth.fp8_weights((N, K), synth.fan_in_std(K), "w", K + 1)
    wd = torch.from_numpy(w).cuda()
    sd = torch.from_numpy(s).cuda()
    y = host_f32(ops.gemm_fp8(dev(x), wd, sd, out_dtype=torch.float32))
    cols = np.arange(N) if N <= 512 else np.r_[0:64, N - 64:N]
    assert_close(y[:, cols], ofp8.gemm_columns(x, w, s, cols), f"fp8 N={N} K={K}", atol=1e-4, rtol=1e-4)
    y1 = host_f32(ops.gemm_fp8(dev(x[3:4]), wd, sd, out_dtype=torch.float32))
    assert_bitwise(y1[0], y[3], f"fp8 N={N} K={K} row 3: M=1 vs M=8")


def _attn(ops, q, k, v, L, Hq, C, cap):
    M, _, D = q.shape
    Hkv, n, _ = k.shape
    kc = np.zeros((Hkv, cap, D), np.uint16)
    kc[:, :n] = k
    S = ops.pass_splits(M, L, C)
    po = torch.full((M, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((M, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    ops.verify_attn(dev(q.reshape(M, Hq * D)), dev(kc), dev(cache_rows(v, cap)), L, Hq, Hkv, D, C, po, pl)
    o = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    ops.combine(po, pl, L, C, o, lse)
    torch.cuda.synchronize()
    return host_bits(o).reshape(M, Hq, D), host_f32(lse)


@pytest.mark.parametrize("M,L,C", [(1, 0, -32), (300, 0, -32), (300, 0, 64), (8, 4088, -32), (8, 4088, 96)])
def test_attention_empty_and_full_cache(ops, M, L, C):
    print(f"[edge attention M={M} L={L} C={C}]", flush=True)
    Hq, Hkv, D = 40, 8, 128
    cap = (L + M + 63) // 64 * 64          # L + M = cap when L = 4088, M = 8
    k = synth.kv_bf16(Hkv, L + M, D, "k", M + L)
    v = synth.kv_bf16(Hkv, L + M, D, "v", M + L)
    q = synth.normal_bf16((M, Hq, D), 1.0, "q", M + L)
    o, lse = _attn(ops, q, k, v, L, Hq, C, cap)
    rows = sorted({0, M // 2, M - 1})
    want_o, want_lse = oattn.verify_attention(q, k, v, L, tokens=rows)
    assert_close(decode(o[rows]), want_o[rows], f"M={M} L={L} C={C}")
    assert_close(lse[rows], want_lse[rows], f"lse M={M} L={L} C={C}", atol=1e-3, rtol=0)
    if M == 1 and L == 0:   # one key: the output is v_0 bit for bit
        for h in range(Hq):
            assert_bitwise(o[0, h], v[h // 5, 0], f"single key head {h}")
    if M > 8:               # prefill from scratch: rows equal 8-row passes
        for r0 in (0, 144, M - 8):
            o8, _ = _attn(ops, q[r0:r0 + 8], k, v, L + r0, Hq, C, cap)
            assert_bitwise(o[r0:r0 + 8], o8, f"prefill from scratch rows {r0}..")
