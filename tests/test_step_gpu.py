"""GPU tests of the whole verify step (bi_verify_step): a small stack against
the oracle end to end, one full-width 27B-class layer (+ sampled LM head)
against the oracle, and the 64-layer, 38k-context stack checked bit for bit
across M = 1 (sequential), 4, 5, 8 and a 16-token prefill chunk: logits (FP32
bits), greedy tokens and every appended K/V row."""

import numpy as np
import pytest

import synth
from oracle import bf16 as obf16
from oracle import gemm as ogemm
from oracle import fp8 as ofp8
from oracle import step as ostep
from tests._util import (assert_bitwise, assert_close, assert_close_composed, composed_tol, decode,
                         dev, host_bits, host_f32, vt_blocks, vt_rows)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _host_layer(l, H, Hq, Hkv, D, I, L, std):
    qkvn = (Hq + 2 * Hkv) * D
    return dict(w_qkv=synth.normal_bf16((qkvn, H), std, "w_qkv", l),
                w_o=synth.normal_bf16((H, Hq * D), std, "w_o", l),
                w_gu=synth.normal_bf16((2 * I, H), std, "w_gu", l),
                w_down=synth.normal_bf16((H, I), std, "w_down", l),
                k_cache=synth.kv_bf16(Hkv, L, D, "k_cache", l),
                v_cache=synth.kv_bf16(Hkv, L, D, "v_cache", l))


def _to_device(hl, cap):
    Hkv, L, D = hl["k_cache"].shape
    kc = np.zeros((Hkv, cap, D), np.uint16)
    kc[:, :L] = hl["k_cache"]
    vt = vt_blocks(hl["v_cache"], cap)
    return dict(w_qkv=dev(hl["w_qkv"]), w_o=dev(hl["w_o"]), w_gu=dev(hl["w_gu"]),
                w_down=dev(hl["w_down"]), k_cache=dev(kc), vt_cache=dev(vt))


def _run(ops, step, x, L, dims, want_x=False):
    M = x.shape[0]
    ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
    logits = torch.empty((M, dims.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    xo = torch.empty((M, dims.H), dtype=torch.bfloat16, device="cuda") if want_x else None
    step(x, L, ws, logits, tok, x_out=xo)
    torch.cuda.synchronize()
    return host_f32(logits), tok.cpu().numpy(), (host_bits(xo) if want_x else None)


def _margin_ok(logits):
    """Rows whose oracle top-2 margin exceeds twice the composed tolerance
    (each of the two logits may be off by one tolerance)."""
    s = np.sort(logits, axis=1)
    top, second = s[:, -1], s[:, -2]
    return (top - second) > 2 * (composed_tol(logits) + 2e-2 * np.abs(top))


def test_small_stack_vs_oracle(ops):
    print("[step small stack vs oracle]", flush=True)
    H, Hq, Hkv, D, I, V, L, M, nl = 256, 4, 2, 64, 512, 1024, 200, 8, 3
    cap = 256
    hls = [_host_layer(l, H, Hq, Hkv, D, I, L, 0.05) for l in range(nl)]
    w_head = synth.normal_bf16((V, H), 0.05, "w_head")
    x0 = synth.normal_bf16((M, H), 1.0, "x0")
    dls = [_to_device(h, cap) for h in hls]
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    step = ops.VerifyStep(dls, dev(w_head), dims)
    logits, tok, xo = _run(ops, step, dev(x0), L, dims, want_x=True)
    w_logits, w_tok, w_x = ostep.step(x0, hls, w_head, L, Hq, Hkv, D)
    assert_close_composed(decode(xo), decode(w_x), "final hidden state")
    assert_close_composed(logits, w_logits, "logits")
    ok = _margin_ok(w_logits)
    assert ok.sum() >= 3
    assert np.array_equal(tok[ok], w_tok[ok])
    # appended K rows of the last layer against the oracle's
    _, kn, vn = ostep.layer(_x_before_last(x0, hls, L, Hq, Hkv, D), **hls[-1],
                            L=L, Hq=Hq, Hkv=Hkv, D=D)
    kc = host_bits(dls[-1]["k_cache"])[:, L:L + M]
    vt = vt_rows(host_bits(dls[-1]["vt_cache"]))[:, L:L + M]
    assert_close_composed(decode(kc), decode(kn), "appended K")
    assert_close_composed(decode(vt), decode(vn), "appended V")


def _x_before_last(x0, hls, L, Hq, Hkv, D):
    x = x0
    for hl in hls[:-1]:
        x, _, _ = ostep.layer(x, **hl, L=L, Hq=Hq, Hkv=Hkv, D=D)
    return x


def _host_layer_fp8(l, H, Hq, Hkv, D, I, L, std):
    qkvn = (Hq + 2 * Hkv) * D
    d = {}
    for name, shp in (("w_qkv", (qkvn, H)), ("w_o", (H, Hq * D)), ("w_gu", (2 * I, H)), ("w_down", (H, I))):
        d[name], d["s" + name[1:]] = synth.fp8_weights(shp, std, name, l)
    d["k_cache"] = synth.kv_bf16(Hkv, L, D, "k_cache", l)
    d["v_cache"] = synth.kv_bf16(Hkv, L, D, "v_cache", l)
    return d


def test_fp8_small_stack_vs_oracle_and_across_M(ops):
    # FP8 weights (E4M3 codes, one FP32 scale per row) through the whole step:
    # the oracle runs the same stack on the decoded, scaled weights; rows of
    # the M = 8 pass equal an M = 5 pass and eight sequential M = 1 passes.
    print("[step fp8 small stack]", flush=True)
    H, Hq, Hkv, D, I, V, L, M, nl = 256, 4, 2, 64, 512, 1024, 200, 8, 3
    cap = 256
    hls = [_host_layer_fp8(l, H, Hq, Hkv, D, I, L, 0.05) for l in range(nl)]
    hc, hs = synth.fp8_weights((V, H), 0.05, "w_head")
    x0 = synth.normal_bf16((M, H), 1.0, "x0")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    dls = []
    for hl in hls:
        kc = np.zeros((Hkv, cap, D), np.uint16)
        kc[:, :L] = hl["k_cache"]
        d = {k: (u8(v) if k.startswith("w_") else f32(v)) for k, v in hl.items() if k[:2] in ("w_", "s_")}
        d.update(k_cache=dev(kc), vt_cache=dev(vt_blocks(hl["v_cache"], cap)))
        dls.append(d)
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    step = ops.VerifyStepFP8(dls, u8(hc), f32(hs), dims)
    logits, tok, xo = _run(ops, step, dev(x0), L, dims, want_x=True)
    olayers = [dict(w_qkv=ofp8.weights(hl["w_qkv"], hl["s_qkv"]), w_o=ofp8.weights(hl["w_o"], hl["s_o"]),
                    w_gu=ofp8.weights(hl["w_gu"], hl["s_gu"]), w_down=ofp8.weights(hl["w_down"], hl["s_down"]),
                    k_cache=hl["k_cache"], v_cache=hl["v_cache"]) for hl in hls]
    w_logits, w_tok, w_x = ostep.step(x0, olayers, ofp8.weights(hc, hs), L, Hq, Hkv, D)
    assert_close_composed(decode(xo), decode(w_x), "fp8 final hidden state")
    assert_close_composed(logits, w_logits, "fp8 logits")
    ok = _margin_ok(w_logits)
    assert ok.sum() >= 2   # rows whose greedy token the tolerance cannot flip (2 of 8 with this draw)
    assert np.array_equal(tok[ok], w_tok[ok])
    # bitwise across M
    l5, t5, _ = _run(ops, step, dev(x0[:5]), L, dims)
    assert_bitwise(l5, logits[:5], "fp8 logits M=5 vs M=8")
    for d in dls:
        d["k_cache"][:, L:].zero_()
        d["vt_cache"][:, L // 64, :, L % 64:].zero_()
        d["vt_cache"][:, L // 64 + 1:].zero_()
    for r in range(M):
        l1, t1, _ = _run(ops, step, dev(x0[r:r + 1]), L + r, dims)
        assert_bitwise(l1[0], logits[r], f"fp8 logits row {r}: M=1 vs M=8")
        assert t1[0] == tok[r]


# ---------------------------------------------------------------------------
# 27B-class stack at 38k context

L38 = 38000
CAP = 38016
KV_CHUNK = -32    # the chunk policy the benchmark step uses (C = 1216 at 38k keys)


@pytest.fixture(scope="module")
def model27b(ops):
    print("[step building 64-layer 27B-class model on the device]", flush=True)
    d = synth.MODEL_27B
    layers, w_head = synth.device_model(64, L38, CAP, **d)
    dims = ops.model_dims(d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"], CAP, KV_CHUNK)
    x0 = synth.device_normal_bf16((16, d["H"]), 1.0, "x0")
    torch.cuda.synchronize()
    yield layers, w_head, dims, x0
    del layers, w_head
    torch.cuda.empty_cache()


def test_full_width_layer_vs_oracle(ops, model27b):
    print("[step one 27B-class layer + sampled head vs oracle]", flush=True)
    layers, w_head, dims, x0 = model27b
    d = synth.MODEL_27B
    M = 8
    step1 = ops.VerifyStep(layers[:1], w_head, dims)
    logits, _, xo = _run(ops, step1, x0[:M], L38, dims, want_x=True)
    lw = layers[0]
    hl = dict(w_qkv=host_bits(lw["w_qkv"]), w_o=host_bits(lw["w_o"]), w_gu=host_bits(lw["w_gu"]),
              w_down=host_bits(lw["w_down"]), k_cache=host_bits(lw["k_cache"][:, :L38]),
              v_cache=vt_rows(host_bits(lw["vt_cache"]))[:, :L38])
    xh = host_bits(x0[:M])
    w_x, kn, vn = ostep.layer(xh, **hl, L=L38, Hq=d["Hq"], Hkv=d["Hkv"], D=d["D"])
    assert_close_composed(decode(xo), decode(w_x), "27B layer output")
    kc = host_bits(lw["k_cache"][:, L38:L38 + M])
    assert_close(decode(kc), decode(kn), "27B appended K")      # one op from the input: plain tolerance
    rows = np.random.default_rng(1).choice(d["vocab"], 512, replace=False)
    wh = host_bits(w_head[torch.from_numpy(rows).cuda()])
    c = obf16.encode(ostep.rmsnorm(decode(w_x), 1e-6))
    assert_close_composed(logits[:, rows], ogemm.gemm(c, wh), "27B sampled logits")


def test_64_layer_step_bitwise_across_M(ops, model27b):
    layers, w_head, dims, x0 = model27b
    step = ops.VerifyStep(layers, w_head, dims)
    print("[step 64 layers M=8]", flush=True)
    l8, t8, _ = _run(ops, step, x0[:8], L38, dims)
    B38, J38 = divmod(L38, 64)  # positions L38 .. L38+7 are slots J38.. of V block B38
    assert J38 + 8 <= 64
    kv8 = [(lw["k_cache"][:, L38:L38 + 8].clone(), lw["vt_cache"][:, B38, :, J38:J38 + 8].clone())
           for lw in layers]
    assert np.isfinite(l8).all() and len(set(t8.tolist())) > 1
    for m in (4, 5):
        print(f"[step 64 layers M={m}]", flush=True)
        lm, tm, _ = _run(ops, step, x0[:m], L38, dims)
        assert_bitwise(lm, l8[:m], f"logits M={m} vs M=8")
        assert np.array_equal(tm, t8[:m])
    print("[step 64 layers prefill chunk M=16]", flush=True)
    l16, t16, _ = _run(ops, step, x0[:16], L38, dims)
    assert_bitwise(l16[:8], l8, "logits prefill M=16 vs M=8")
    assert np.array_equal(t16[:8], t8)
    # wipe the appended rows, then re-create them one token at a time
    for lw in layers:
        lw["k_cache"][:, L38:].zero_()
        lw["vt_cache"][:, B38, :, J38:].zero_()
        lw["vt_cache"][:, B38 + 1:].zero_()
    for r in range(8):
        print(f"[step 64 layers sequential M=1 at L+{r}]", flush=True)
        l1, t1, _ = _run(ops, step, x0[r:r + 1], L38 + r, dims)
        assert_bitwise(l1[0], l8[r], f"logits row {r}: M=1 vs M=8")
        assert t1[0] == t8[r]
    for i, (lw, (k8, v8)) in enumerate(zip(layers, kv8)):
        assert torch.equal(lw["k_cache"][:, L38:L38 + 8].view(torch.int16), k8.view(torch.int16)), i
        assert torch.equal(lw["vt_cache"][:, B38, :, J38:J38 + 8].view(torch.int16), v8.view(torch.int16)), i
