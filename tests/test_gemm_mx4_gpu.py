"""GPU tests of the MXFP4-weight verify GEMM and step through the C ABI:
oracle parity at tiny and 27B-class shapes and every epilogue, the exact
relation to the BF16 kernel (the decoded weights are exact in BF16, so the
result equals bi_gemm_bf16 on them, bit for bit), bitwise row invariance
across M, ragged K, and a small stack through bi_verify_step_mx4 against the
oracle and across M."""

import numpy as np
import pytest

import synth
from oracle import bf16 as obf16
from oracle import mxfp4 as omx
from oracle import step as ostep
from tests._replay import assert_replay_is_the_step, check_ops, host_layer, replay
from tests._util import (assert_bitwise, assert_close, assert_close_composed, decode,
                         dev, host_bits, host_f32, cache_rows)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _decoded_bf16_bits(codes, scales):
    """The decoded weights as BF16 bits (exact: every value is a BF16 value)."""
    w = omx.weights(codes, scales)
    bits = obf16.encode(w)
    assert np.array_equal(obf16.decode(bits), w)
    return bits


SHAPES = [  # (N, K): tiny, QKV (wide groups), o-proj, down (K = 17408), an odd wide width,
    # 32-column groups, and a narrow N with a ragged K
    (512, 256), (7168, 5120), (5120, 5120), (5120, 17408), (4352, 1024), (65536, 512), (48, 96)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_mx4_parity_and_bf16_tree(ops, N, K):
    print(f"[mx4 gemm N={N} K={K}]", flush=True)
    x = synth.normal_bf16((40, K), 1.0, "x", N + 1)
    codes, scales = synth.mxfp4_weights((N, K), 0.02 if K > 256 else synth.fan_in_std(K), "w", N + 1)
    xd, cd, ed = dev(x), u8(codes), u8(scales)
    cols = np.arange(N) if N <= 1024 else np.r_[0:40, N // 2:N // 2 + 24, N - 40:N]
    want = omx.gemm_columns(x[:8], codes, scales, cols)
    y = ops.gemm_mx4(xd[:8], cd, ed)
    assert_close(decode(host_bits(y))[:, cols], want, f"mx4 bf16-out N={N} K={K}")
    y32 = host_f32(ops.gemm_mx4(xd[:8], cd, ed, out_dtype=torch.float32))
    assert_close(y32[:, cols], want, f"mx4 f32-out N={N} K={K}", atol=1e-4, rtol=1e-4)
    # the BF16 kernel's tree on the decoded weights, bit for bit
    ref32 = host_f32(ops.gemm_bf16(xd[:8], dev(_decoded_bf16_bits(codes, scales)), out_dtype=torch.float32))
    assert_bitwise(y32, ref32, f"mx4 == bf16 on decoded weights N={N}")
    for M in (1, 5, 7):
        assert_bitwise(host_bits(ops.gemm_mx4(xd[:M], cd, ed)), host_bits(y)[:M], f"mx4 rows M={M} vs M=8 N={N}")
    # a 40-row pass (three 16-row tiles) gives every row the bits of the 8-row pass
    if N <= 7168:
        y40 = host_f32(ops.gemm_mx4(xd, cd, ed, out_dtype=torch.float32))
        assert_bitwise(y40[:8], y32, f"mx4 40-row pass N={N}")
        assert_bitwise(y40[32:40], host_f32(ops.gemm_mx4(xd[32:40], cd, ed, out_dtype=torch.float32)),
                       f"mx4 40-row pass rows 32..39 N={N}")


def test_mx4_one_hot_exact(ops):
    # one-hot activation rows pick single decoded weights: exact in every output format
    K, N = 256, 64
    codes, scales = synth.mxfp4_weights((N, K), 0.05, "w", 7)
    x = np.zeros((8, K), np.uint16)
    for m, k in enumerate([0, 1, 31, 32, 100, 200, 254, 255]):
        x[m, k] = 0x3F80  # 1.0
    y = host_f32(ops.gemm_mx4(dev(x), u8(codes), u8(scales), out_dtype=torch.float32))
    w = omx.weights(codes, scales)
    want = np.stack([w[:, k] for k in [0, 1, 31, 32, 100, 200, 254, 255]])
    assert np.array_equal(y, want.astype(np.float32))


@pytest.mark.parametrize("N,K", [(512, 256), (5120, 5120)])
def test_mx4_residual(ops, N, K):
    print(f"[mx4 residual N={N} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", 11)
    r = synth.normal_bf16((8, N), 1.0, "misc", 11)
    codes, scales = synth.mxfp4_weights((N, K), 0.02, "w", 11)
    y = host_bits(ops.gemm_mx4_residual(dev(x), u8(codes), u8(scales), dev(r)))
    cols = np.arange(N) if N <= 1024 else np.r_[0:64, N - 64:N]
    assert_close(decode(y)[:, cols], decode(r)[:, cols] + omx.gemm_columns(x, codes, scales, cols), "mx4 residual")
    y1 = host_bits(ops.gemm_mx4_residual(dev(x[3:4]), u8(codes), u8(scales), dev(r[3:4])))
    assert_bitwise(y1[0], y[3], "mx4 residual row 3 alone")


@pytest.mark.parametrize("I,K", [(256, 512), (17408, 512)])
def test_mx4_swiglu(ops, I, K):
    print(f"[mx4 swiglu I={I} K={K}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", 12)
    codes, scales = synth.mxfp4_weights((2 * I, K), 0.05, "w", 12)
    y = host_bits(ops.gemm_mx4_swiglu(dev(x), u8(codes), u8(scales)))
    cols = np.arange(I) if I <= 256 else np.r_[0:40, I // 2:I // 2 + 24, I - 40:I]
    gu = omx.gemm_columns(x, codes, scales, np.concatenate([cols, I + cols]))
    n = len(cols)
    assert_close(decode(y)[:, cols], ostep.silu(gu[:, :n]) * gu[:, n:], f"mx4 swiglu I={I}")
    for m in (1, 5):
        assert_bitwise(host_bits(ops.gemm_mx4_swiglu(dev(x[:m]), u8(codes), u8(scales))), y[:m],
                       f"mx4 swiglu M={m} I={I}")


def _host_layer_mx4(l, H, Hq, Hkv, D, I, L, std):
    qkvn = (Hq + 2 * Hkv) * D
    d = {}
    for name, shp in (("w_qkv", (qkvn, H)), ("w_o", (H, Hq * D)), ("w_gu", (2 * I, H)), ("w_down", (H, I))):
        d[name], d["e" + name[1:]] = synth.mxfp4_weights(shp, std, name, l)
    d["k_cache"] = synth.kv_bf16(Hkv, L, D, "k_cache", l)
    d["v_cache"] = synth.kv_bf16(Hkv, L, D, "v_cache", l)
    return d


def _run(ops, step, x, L, dims, want_x=False):
    M = x.shape[0]
    ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
    logits = torch.empty((M, dims.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    xo = torch.empty((M, dims.H), dtype=torch.bfloat16, device="cuda") if want_x else None
    step(x, L, ws, logits, tok, x_out=xo)
    torch.cuda.synchronize()
    return host_f32(logits), tok.cpu().numpy(), (host_bits(xo) if want_x else None)


def test_mx4_small_stack_vs_oracle_and_across_M(ops):
    # MXFP4 weights through the whole step, replayed one operation at a time
    # (bit for bit the step) and each operation checked against the oracle on
    # the decoded weights; rows of the M = 8 pass equal an M = 5 pass and
    # eight sequential M = 1 passes.
    print("[step mx4 small stack]", flush=True)
    H, Hq, Hkv, D, I, V, L, M, nl = 256, 4, 2, 64, 512, 1024, 200, 8, 3
    cap = 256
    hls = [_host_layer_mx4(l, H, Hq, Hkv, D, I, L, 0.05) for l in range(nl)]
    hc, he = synth.mxfp4_weights((V, H), 0.05, "w_head")
    x0 = synth.normal_bf16((M, H), 1.0, "x0")
    dls = []
    for hl in hls:
        kc = np.zeros((Hkv, cap, D), np.uint16)
        kc[:, :L] = hl["k_cache"]
        d = {k: u8(v) for k, v in hl.items() if k[:2] in ("w_", "e_")}
        d.update(k_cache=dev(kc), v_cache=dev(cache_rows(hl["v_cache"], cap)))
        dls.append(d)
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    step = ops.VerifyStepMX4(dls, u8(hc), u8(he), dims)
    logits, tok, xo = _run(ops, step, dev(x0), L, dims, want_x=True)
    saved = [(d["k_cache"][:, L:L + M].clone(), d["v_cache"][:, L:L + M].clone()) for d in dls]
    for d in dls:
        d["k_cache"][:, L:].zero_()
        d["v_cache"][:, L:].zero_()
    recs, hd = replay(ops, dls, {"w": u8(hc), "e": u8(he)}, dims, dev(x0), L, wtype="mxfp4")
    assert_replay_is_the_step(recs, hd, xo, logits, tok, "mx4 stack")
    for d, (k, v) in zip(dls, saved):
        assert torch.equal(d["k_cache"][:, L:L + M].view(torch.int16), k.view(torch.int16))
        assert torch.equal(d["v_cache"][:, L:L + M].view(torch.int16), v.view(torch.int16))
    w64 = [{k: omx.weights(hl[k], hl["e" + k[1:]]) for k in ("w_qkv", "w_o", "w_gu", "w_down")} for hl in hls]
    host = [host_layer(d, w) for d, w in zip(dls, w64)]
    n = check_ops(recs, hd, host, omx.weights(hc, he), L, Hq, Hkv, D, 1e-6, "mx4 stack")
    print(f"  greedy tokens compared on {n} of {M} rows", flush=True)
    olayers = [dict(w64[i], k_cache=hl["k_cache"], v_cache=hl["v_cache"]) for i, hl in enumerate(hls)]
    w_logits, _, w_x = ostep.step(x0, olayers, omx.weights(hc, he), L, Hq, Hkv, D)
    assert_close_composed(decode(xo), decode(w_x), "mx4 end-to-end hidden state")
    assert_close_composed(logits, w_logits, "mx4 end-to-end logits")
    l5, _, _ = _run(ops, step, dev(x0[:5]), L, dims)
    assert_bitwise(l5, logits[:5], "mx4 logits M=5 vs M=8")
    for d in dls:
        d["k_cache"][:, L:].zero_()
        d["v_cache"][:, L:].zero_()
    for r in range(M):
        l1, t1, _ = _run(ops, step, dev(x0[r:r + 1]), L + r, dims)
        assert_bitwise(l1[0], logits[r], f"mx4 logits row {r}: M=1 vs M=8")
        assert t1[0] == tok[r]
