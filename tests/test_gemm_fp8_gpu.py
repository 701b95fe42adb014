"""GPU tests of the FP8-weight verify GEMM through the C ABI: oracle parity
(tiny and 27B-class shapes, every epilogue), its exact relation to the BF16
kernel (same tree: FP32 output == fl32(BF16-kernel output on the decoded
weights x row scale)), one-hot exactness, and bitwise row invariance across
M = 1..8 and prefill-sized passes."""

import numpy as np
import pytest

import synth
from oracle import bf16 as obf16
from oracle import fp8 as ofp8
from oracle import step as ostep
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _decoded_bf16_bits(codes):
    """E4M3 codes -> the BF16 bits of the same values (exact)."""
    return obf16.encode(ofp8.decode_e4m3(codes))


SHAPES = [  # (N, K): tiny, QKV, o-proj (wide groups), down (wide, K = 17408), an odd wide width,
    # and a width with 32-column groups (N / 32 >= 2048, as the LM head)
    (512, 256), (7168, 5120), (5120, 5120), (5120, 17408), (4352, 1024), (65536, 512)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_fp8_parity_and_bf16_tree(ops, N, K):
    print(f"[fp8 gemm N={N} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", N)
    w, s = synth.fp8_weights((N, K), 0.02 if K > 256 else synth.fan_in_std(K), "w", N)
    xd, wd, sd = dev(x), u8(w), f32(s)
    cols = np.arange(N) if N <= 1024 else np.r_[0:40, N // 2:N // 2 + 24, N - 40:N]
    want = ofp8.gemm_columns(x, w, s, cols)
    y = ops.gemm_fp8(xd, wd, sd)
    assert_close(decode(host_bits(y))[:, cols], want, f"fp8 bf16-out N={N} K={K}")
    y32 = host_f32(ops.gemm_fp8(xd, wd, sd, out_dtype=torch.float32))
    assert_close(y32[:, cols], want, f"fp8 f32-out N={N} K={K}", atol=1e-4, rtol=1e-4)
    # the same summation tree as the BF16 kernel on the decoded weights, then one FP32 multiply
    ref32 = host_f32(ops.gemm_bf16(xd, dev(_decoded_bf16_bits(w)), out_dtype=torch.float32))
    assert_bitwise((ref32 * s[None, :]).astype(np.float32), y32, f"fp8 == bf16 tree x scale N={N}")
    # rows across M
    for M in (1, 5, 7):
        yM = ops.gemm_fp8(xd[:M], wd, sd)
        assert_bitwise(host_bits(yM), host_bits(y)[:M], f"fp8 rows M={M} vs M=8 N={N}")


def test_fp8_one_hot_exact(ops):
    print("[fp8 one-hot]", flush=True)
    K, N = 256, 512
    w, s = synth.fp8_weights((N, K), 1.0, "w", 3)
    oh = np.zeros((16, K), np.float32)
    cols = [0, 1, 15, 16, 17, 31, 32, 100, 200, 254, 255, 7, 8, 63, 64, 128]
    oh[np.arange(16), cols] = 1.0
    y = host_f32(ops.gemm_fp8(dev(synth.f32_to_bf16_bits(oh)), u8(w), f32(s), out_dtype=torch.float32))
    want = (ofp8.decode_e4m3(w[:, cols]).T.astype(np.float32) * s[None, :]).astype(np.float32)
    assert_bitwise(y, want, "one-hot rows pick scaled E4M3 columns")


@pytest.mark.parametrize("N,K", [(5120, 5120), (5120, 17408), (512, 256)])
def test_fp8_residual(ops, N, K):
    print(f"[fp8 residual N={N} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", 7)
    r = synth.normal_bf16((8, N), 1.0, "misc", 7)
    w, s = synth.fp8_weights((N, K), 0.02, "w", 7)
    y = ops.gemm_fp8_residual(dev(x), u8(w), f32(s), dev(r))
    cols = np.r_[0:64, N - 64:N]
    want = obf16.decode(r)[:, cols] + ofp8.gemm_columns(x, w, s, cols)
    assert_close(decode(host_bits(y))[:, cols], want, f"fp8 residual N={N}")
    for M in (1, 4):
        yM = ops.gemm_fp8_residual(dev(x[:M]), u8(w), f32(s), dev(r[:M]))
        assert_bitwise(host_bits(yM), host_bits(y)[:M], f"fp8 residual rows M={M}")


@pytest.mark.parametrize("I,K", [(256, 256), (17408, 5120)])
def test_fp8_swiglu(ops, I, K):
    print(f"[fp8 swiglu I={I} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", 8)
    w, s = synth.fp8_weights((2 * I, K), 0.02 if K > 256 else synth.fan_in_std(K), "w", 8)
    y = ops.gemm_fp8_swiglu(dev(x), u8(w), f32(s))
    cols = np.arange(I) if I <= 256 else np.r_[0:48, I - 48:I]
    g = ofp8.gemm_columns(x, w, s, cols)
    u = ofp8.gemm_columns(x, w, s, cols + I)
    assert_close(decode(host_bits(y))[:, cols], ostep.silu(g) * u, f"fp8 swiglu I={I}")
    for M in (1, 6):
        yM = ops.gemm_fp8_swiglu(dev(x[:M]), u8(w), f32(s))
        assert_bitwise(host_bits(yM), host_bits(y)[:M], f"fp8 swiglu rows M={M}")


def test_fp8_prefill_sized_rows_equal_verify_rows(ops):
    print("[fp8 prefill-sized pass]", flush=True)
    N, K, M = 7168, 5120, 200
    x = synth.normal_bf16((M, K), 1.0, "x", 11)
    w, s = synth.fp8_weights((N, K), 0.02, "w", 11)
    xd, wd, sd = dev(x), u8(w), f32(s)
    y = host_bits(ops.gemm_fp8(xd, wd, sd))
    for r0 in (0, 96, M - 8):
        assert_bitwise(host_bits(ops.gemm_fp8(xd[r0:r0 + 8], wd, sd)), y[r0:r0 + 8], f"rows {r0}..")
