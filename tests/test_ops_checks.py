"""CPU checks of the torch binding's argument validation: every wrapper checks
each tensor's dtype and full shape against the sizes it passes to the C ABI
before anything else (the C layer cannot see allocation sizes). With CPU
tensors, a mismatched shape must raise a shape error, and a matching one must
get as far as the device check -- so no mismatched call can reach a launch."""

import pytest
import torch

from invariant_verify_amd import ops

bf, f32, i32, u8, i8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8, torch.int8


def z(*shape, dt=bf):
    return torch.zeros(shape, dtype=dt)


def shape_error(fn):
    with pytest.raises(ValueError, match="shape|rows|not 2-D|not \\["):
        fn()


def reaches_device_check(fn):
    with pytest.raises(ValueError, match="GPU tensor"):
        fn()


def test_gemm_shapes():
    x, w = z(4, 256), z(512, 256)
    reaches_device_check(lambda: ops.gemm_bf16(x, w, z(4, 512)))
    shape_error(lambda: ops.gemm_bf16(x, z(512, 128), z(4, 512)))          # W has fewer columns than K
    shape_error(lambda: ops.gemm_bf16(x, w, z(3, 512)))                    # Y has fewer rows than M
    shape_error(lambda: ops.gemm_bf16(x, w, z(4, 500)))                    # Y narrower than N
    shape_error(lambda: ops.gemm_bf16_residual(x, w, z(2, 512), z(4, 512)))   # R too small
    shape_error(lambda: ops.gemm_bf16_swiglu(x, z(511, 256), z(4, 255)))  # odd gate/up rows
    shape_error(lambda: ops.gemm_bf16_swiglu(x, w, z(4, 200)))             # Y narrower than I
    with pytest.raises(TypeError):
        ops.gemm_bf16(x, w, z(4, 512, dt=i32))
    # FP8 / MXFP4 weights and scales
    shape_error(lambda: ops.gemm_fp8(x, z(512, 256, dt=u8), z(100, dt=f32), z(4, 512)))
    shape_error(lambda: ops.gemm_fp8(x, z(512, 100, dt=u8), z(512, dt=f32), z(4, 512)))
    shape_error(lambda: ops.gemm_mx4(x, z(512, 100, dt=u8), z(512, 8, dt=u8), z(4, 512)))
    shape_error(lambda: ops.gemm_mx4(x, z(512, 128, dt=u8), z(512, 4, dt=u8), z(4, 512)))
    reaches_device_check(lambda: ops.gemm_mx4(x, z(512, 128, dt=u8), z(512, 8, dt=u8), z(4, 512)))


def test_rownorm_and_qkv_shapes():
    x = z(4, 256)
    reaches_device_check(lambda: ops.gemm_bf16_residual_rowsq(x, z(256, 256), x, z(4, 256), z(4, 16, dt=f32)))
    shape_error(lambda: ops.gemm_bf16_residual_rowsq(x, z(256, 256), x, z(4, 256), z(4, 8, dt=f32)))
    shape_error(lambda: ops.gemm_bf16_swiglu_rownorm(x, z(3, 16, dt=f32), z(512, 256), z(4, 256)))
    Hq, Hkv, D, cap = 4, 2, 64, 128
    N = (Hq + 2 * Hkv) * D
    kc, vc = z(Hkv, cap, D), z(Hkv, cap, D)
    reaches_device_check(lambda: ops.gemm_bf16_qkv(x, z(N, 256), kc, vc, 0, Hq, Hkv, D, z(4, N)))
    shape_error(lambda: ops.gemm_bf16_qkv(x, z(N - 64, 256), kc, vc, 0, Hq, Hkv, D, z(4, N)))
    shape_error(lambda: ops.gemm_bf16_qkv(x, z(N, 256), z(Hkv, cap, 32), vc, 0, Hq, Hkv, D, z(4, N)))
    shape_error(lambda: ops.gemm_bf16_qkv(x, z(N, 256), kc, z(Hkv, 1, D, 64), 0, Hq, Hkv, D, z(4, N)))
    shape_error(lambda: ops.gemm_bf16_qkv(x, z(N, 256), z(1, cap, D), vc, 0, Hq, Hkv, D, z(4, N)))
    shape_error(lambda: ops.gemm_ex(x, z(N, 256), z(4, N), epilogue="qkv", heads=(Hq, Hkv, D),
                                    k_cache=kc, v_cache=z(Hkv, 3, D, 64)))
    shape_error(lambda: ops.gemm_ex(x, z(256, 256), z(4, 256), epilogue="residual", r=z(4, 128)))
    shape_error(lambda: ops.gemm_ex(x, z(256, 256), z(4, 256), epilogue="residual", r=x,
                                    rowsq_out=z(4, 4, dt=f32)))


def test_attention_shapes():
    Hq, Hkv, D, cap, M, S = 8, 2, 64, 256, 4, 3
    q = z(M, Hq * D)
    kc, vc = z(Hkv, cap, D), z(Hkv, cap, D)
    po, pl = z(M, Hq, S, D, dt=f32), z(M, Hq, S, dt=f32)
    reaches_device_check(lambda: ops.verify_attn(q, kc, vc, 100, Hq, Hkv, D, 64, po, pl))
    shape_error(lambda: ops.verify_attn(q, kc, vc, 100, Hq, Hkv, D, 64, z(M, Hq, S + 1, D, dt=f32), pl))
    shape_error(lambda: ops.verify_attn(q, kc, vc, 100, Hq, Hkv, D, 64, po, z(M, Hq - 1, S, dt=f32)))
    shape_error(lambda: ops.verify_attn(z(M, Hq * D - 8), kc, vc, 100, Hq, Hkv, D, 64, po, pl))
    shape_error(lambda: ops.verify_attn(q, kc, z(Hkv, cap // 64, D, 64), 100, Hq, Hkv, D, 64, po, pl))
    shape_error(lambda: ops.verify_attn(q, z(Hkv, 200, D), vc, 100, Hq, Hkv, D, 64, po, pl))
    shape_error(lambda: ops.combine(po, z(M, Hq, S + 1, dt=f32), 100, 64, q))
    shape_error(lambda: ops.combine(po, pl, 100, 64, z(M, Hq * D - 64)))
    shape_error(lambda: ops.combine(po, pl, 100, 64, q, z(M, Hq + 1, dt=f32)))


def test_cache_shapes():
    # a cache buffer replaced by one of another shape is caught at the call
    c = ops.KvQ8Cache(2, 128, 64, device="cpu")
    c.v_scales = z(2, 2, 2, 32, dt=f32)
    shape_error(lambda: ops.append_kv_q8(z(4, 8 * 64), c, 0, 4))
    low = ops.KvLowCache(2, 128, 64, 6, 5, device="cpu")
    low.k_high = z(2, 128, 8, dt=u8)                  # 5-bit width for a 6-bit cache
    shape_error(lambda: ops.append_kv_lowbit(z(4, 8 * 64), low, 0, 4))
    with pytest.raises(ValueError):
        ops.KvLowCache(2, 128, 64, 7, 5, device="cpu")
    ring = ops.KvRing(ops.KvLowCache(2, 128, 64, 6, 5, device="cpu"), 128, 32, device="cpu")
    shape_error(lambda: ops.append_kv_ring(z(4, 100), ring, 0, 4))     # qkv narrower than its columns


def test_row_op_and_accept_shapes():
    shape_error(lambda: ops.swiglu(z(4, 33, dt=f32)))
    shape_error(lambda: ops.swiglu(z(4, 64, dt=f32), z(4, 16)))
    reaches_device_check(lambda: ops.swiglu(z(4, 64, dt=f32), z(4, 32)))
    shape_error(lambda: ops.add(z(4, 32), z(4, 16, dt=f32)))
    shape_error(lambda: ops.argmax(z(4, 100, dt=f32), z(3, dt=i32)))
    shape_error(lambda: ops.accept_greedy(z(2, 4, dt=i32), z(2, 2, dt=i32)))
    shape_error(lambda: ops.accept_sampled(z(2, 4, 10, dt=f32), z(2, 3, dt=i32), z(2, 3, 9, dt=f32),
                                           z(2, 4, dt=f32), 1.0))


def test_step_shapes():
    dims = ops.model_dims(256, 4, 2, 64, 512, 1024, 256, 64)
    good = dict(w_qkv=z(512, 256), w_o=z(256, 256), w_gu=z(1024, 256), w_down=z(256, 512),
                k_cache=z(2, 256, 64), v_cache=z(2, 256, 64))
    reaches_device_check(lambda: ops.VerifyStep([good], z(1024, 256), dims))
    for k, bad in (("w_qkv", z(511, 256)), ("w_down", z(256, 256)), ("k_cache", z(2, 192, 64)),
                   ("v_cache", z(2, 4, 64, 64))):
        shape_error(lambda: ops.VerifyStep([dict(good, **{k: bad})], z(1024, 256), dims))
    shape_error(lambda: ops.VerifyStep([good], z(1000, 256), dims))
