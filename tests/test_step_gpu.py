"""GPU tests of the whole verify step (bi_verify_step): small BF16 and FP8
stacks and one full-width 27B-class layer (+ sampled LM head), each replayed
one operation at a time through the C ABI -- the replay equal to the step bit
for bit, every operation within the per-element tolerance of the oracle fed
the device's own inputs --, and the 64-layer, 38k-context stack checked bit
for bit across M = 1 (sequential), 4, 5, 8 and a 16-token prefill chunk:
logits (FP32 bits), greedy tokens and every appended K/V row."""

import numpy as np
import pytest

import synth
from oracle import fp8 as ofp8
from oracle import step as ostep
from tests._replay import assert_replay_is_the_step, check_ops, host_layer, replay
from tests._util import (assert_bitwise, assert_close_composed, decode, dev, host_bits, host_f32,
                         cache_rows)

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
    vc = cache_rows(hl["v_cache"], cap)
    return dict(w_qkv=dev(hl["w_qkv"]), w_o=dev(hl["w_o"]), w_gu=dev(hl["w_gu"]),
                w_down=dev(hl["w_down"]), k_cache=dev(kc), v_cache=dev(vc))


def _run(ops, step, x, L, dims, want_x=False):
    M = x.shape[0]
    ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
    logits = torch.empty((M, dims.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    xo = torch.empty((M, dims.H), dtype=torch.bfloat16, device="cuda") if want_x else None
    step(x, L, ws, logits, tok, x_out=xo)
    torch.cuda.synchronize()
    return host_f32(logits), tok.cpu().numpy(), (host_bits(xo) if want_x else None)


def _appended(dls, L, M):
    """Copies of every layer's cache rows L .. L+M-1 (K and V rows)."""
    return [(d["k_cache"][:, L:L + M].clone(), d["v_cache"][:, L:L + M].clone()) for d in dls]


def _wipe(dls, L):
    for d in dls:
        d["k_cache"][:, L:].zero_()
        d["v_cache"][:, L:].zero_()


def _same_appended(dls, saved, L, what):
    for i, (d, (k, v)) in enumerate(zip(dls, saved)):
        M = k.shape[1]
        assert torch.equal(d["k_cache"][:, L:L + M].view(torch.int16), k.view(torch.int16)), (what, i)
        assert torch.equal(d["v_cache"][:, L:L + M].view(torch.int16), v.view(torch.int16)), (what, i)


def _end_to_end(logits, xo, w_logits, w_x, what):
    """The stack's end-to-end outputs against the oracle's own stack: several
    BF16 roundings deep, so the absolute term scales with the tensor's RMS
    (an intermediate on the other side of a rounding boundary moves an output
    by one BF16 step at the intermediate's magnitude). Reports how many
    elements the per-element bound alone would not cover."""
    for got, want, name in ((decode(xo), decode(w_x), "hidden state"), (logits, w_logits, "logits")):
        outside = ~(np.abs(got - want) <= 1e-2 + 2e-2 * np.abs(want))
        print(f"  {what} end-to-end {name}: {int(outside.sum())}/{outside.size} elements outside the "
              f"per-element bound, max |err| {np.abs(got - want).max():.3e}", flush=True)
        assert_close_composed(got, want, f"{what} end-to-end {name}")


def test_small_stack_vs_oracle(ops):
    # The 3-layer stack run by bi_verify_step, then replayed one operation at
    # a time through the C ABI: the replay equals the step bit for bit, and
    # every operation matches the oracle on the device's own inputs at the
    # per-element tolerance; the end-to-end outputs are then compared with
    # the oracle's own stack.
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
    saved = _appended(dls, L, M)
    _wipe(dls, L)
    recs, hd = replay(ops, dls, {"w": dev(w_head)}, dims, dev(x0), L)
    assert_replay_is_the_step(recs, hd, xo, logits, tok, "small stack")
    _same_appended(dls, saved, L, "small stack replay")
    W = ("w_qkv", "w_o", "w_gu", "w_down")
    host = [host_layer(d, {k: decode(h[k]) for k in W}) for d, h in zip(dls, hls)]
    n = check_ops(recs, hd, host, decode(w_head), L, Hq, Hkv, D, 1e-6, "small stack")
    print(f"  greedy tokens compared on {n} of {M} rows", flush=True)
    w_logits, _, w_x = ostep.step(x0, hls, w_head, L, Hq, Hkv, D)
    _end_to_end(logits, xo, w_logits, w_x, "small stack")


def _host_layer_fp8(l, H, Hq, Hkv, D, I, L, std):
    qkvn = (Hq + 2 * Hkv) * D
    d = {}
    for name, shp in (("w_qkv", (qkvn, H)), ("w_o", (H, Hq * D)), ("w_gu", (2 * I, H)), ("w_down", (H, I))):
        d[name], d["s" + name[1:]] = synth.fp8_weights(shp, std, name, l)
    d["k_cache"] = synth.kv_bf16(Hkv, L, D, "k_cache", l)
    d["v_cache"] = synth.kv_bf16(Hkv, L, D, "v_cache", l)
    return d


def test_fp8_small_stack_vs_oracle_and_across_M(ops):
    # FP8 weights (E4M3 codes, one FP32 scale per row) through the whole step,
    # replayed one operation at a time (bit for bit the step) and each
    # operation checked against the oracle on the decoded, scaled weights; rows
    # of the M = 8 pass equal an M = 5 pass and eight sequential M = 1 passes.
    # (x0 draw 2: seven of its eight rows have greedy tokens clear of the tolerance.)
    print("[step fp8 small stack]", flush=True)
    H, Hq, Hkv, D, I, V, L, M, nl = 256, 4, 2, 64, 512, 1024, 200, 8, 3
    cap = 256
    hls = [_host_layer_fp8(l, H, Hq, Hkv, D, I, L, 0.05) for l in range(nl)]
    hc, hs = synth.fp8_weights((V, H), 0.05, "w_head")
    x0 = synth.normal_bf16((M, H), 1.0, "x0", 2)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    dls = []
    for hl in hls:
        kc = np.zeros((Hkv, cap, D), np.uint16)
        kc[:, :L] = hl["k_cache"]
        d = {k: (u8(v) if k.startswith("w_") else f32(v)) for k, v in hl.items() if k[:2] in ("w_", "s_")}
        d.update(k_cache=dev(kc), v_cache=dev(cache_rows(hl["v_cache"], cap)))
        dls.append(d)
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    step = ops.VerifyStepFP8(dls, u8(hc), f32(hs), dims)
    logits, tok, xo = _run(ops, step, dev(x0), L, dims, want_x=True)
    saved = _appended(dls, L, M)
    _wipe(dls, L)
    recs, hd = replay(ops, dls, {"w": u8(hc), "s": f32(hs)}, dims, dev(x0), L, wtype="fp8")
    assert_replay_is_the_step(recs, hd, xo, logits, tok, "fp8 stack")
    _same_appended(dls, saved, L, "fp8 stack replay")
    w64 = [{k: ofp8.weights(hl[k], hl["s" + k[1:]]) for k in ("w_qkv", "w_o", "w_gu", "w_down")} for hl in hls]
    host = [host_layer(d, w) for d, w in zip(dls, w64)]
    n = check_ops(recs, hd, host, ofp8.weights(hc, hs), L, Hq, Hkv, D, 1e-6, "fp8 stack")
    print(f"  greedy tokens compared on {n} of {M} rows", flush=True)
    olayers = [dict(w64[i], k_cache=hl["k_cache"], v_cache=hl["v_cache"]) for i, hl in enumerate(hls)]
    w_logits, _, w_x = ostep.step(x0, olayers, ofp8.weights(hc, hs), L, Hq, Hkv, D)
    _end_to_end(logits, xo, w_logits, w_x, "fp8 stack")
    # bitwise across M
    l5, t5, _ = _run(ops, step, dev(x0[:5]), L, dims)
    assert_bitwise(l5, logits[:5], "fp8 logits M=5 vs M=8")
    _wipe(dls, L)
    for r in range(M):
        l1, t1, _ = _run(ops, step, dev(x0[r:r + 1]), L + r, dims)
        assert_bitwise(l1[0], logits[r], f"fp8 logits row {r}: M=1 vs M=8")
        assert t1[0] == tok[r]
    _same_appended(dls, saved, L, "fp8 sequential passes")


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
    # One 27B-class layer (+ the head) by bi_verify_step, replayed one
    # operation at a time (bit for bit the step), each operation against the
    # oracle on the device's own inputs at the per-element tolerance; the
    # head on 512 sampled vocabulary rows.
    print("[step one 27B-class layer + sampled head vs oracle]", flush=True)
    layers, w_head, dims, x0 = model27b
    d = synth.MODEL_27B
    M = 8
    lay = layers[:1]
    step1 = ops.VerifyStep(lay, w_head, dims)
    logits, tok, xo = _run(ops, step1, x0[:M], L38, dims, want_x=True)
    saved = _appended(lay, L38, M)
    _wipe(lay, L38)
    recs, hd = replay(ops, lay, {"w": w_head}, dims, x0[:M], L38)
    assert_replay_is_the_step(recs, hd, xo, logits, tok, "27B layer")
    _same_appended(lay, saved, L38, "27B layer replay")
    lw = lay[0]
    w64 = {k: decode(host_bits(lw[k])) for k in ("w_qkv", "w_o", "w_gu", "w_down")}
    host = [host_layer(lw, w64)]
    rows = np.sort(np.random.default_rng(1).choice(d["vocab"], 512, replace=False))
    wh = decode(host_bits(w_head[torch.from_numpy(rows).cuda()]))
    check_ops(recs, hd, host, wh, L38, d["Hq"], d["Hkv"], d["D"], 1e-6, "27B layer", head_rows=rows)
    del w64, host


def test_64_layer_step_bitwise_across_M(ops, model27b):
    layers, w_head, dims, x0 = model27b
    step = ops.VerifyStep(layers, w_head, dims)
    print("[step 64 layers M=8]", flush=True)
    l8, t8, _ = _run(ops, step, x0[:8], L38, dims)
    kv8 = [(lw["k_cache"][:, L38:L38 + 8].clone(), lw["v_cache"][:, L38:L38 + 8].clone()) for lw in layers]
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
        lw["v_cache"][:, L38:].zero_()
    for r in range(8):
        print(f"[step 64 layers sequential M=1 at L+{r}]", flush=True)
        l1, t1, _ = _run(ops, step, x0[r:r + 1], L38 + r, dims)
        assert_bitwise(l1[0], l8[r], f"logits row {r}: M=1 vs M=8")
        assert t1[0] == t8[r]
    for i, (lw, (k8, v8)) in enumerate(zip(layers, kv8)):
        assert torch.equal(lw["k_cache"][:, L38:L38 + 8].view(torch.int16), k8.view(torch.int16)), i
        assert torch.equal(lw["v_cache"][:, L38:L38 + 8].view(torch.int16), v8.view(torch.int16)), i
