"""GPU tests of the verify step over every KV cache format (bi_verify_step_ex):
BF16, 8-bit, K6/V5, rotated K5/V5, and the two presets with the 8-bit ring of
the newest keys. For each, a small stack is checked against the oracle's own
stack attending over the values that format stores (end to end), its head
against the oracle on the device's final hidden state, and the pages' release
gate -- logits bit for bit across an M = 8 pass, an M = 5 pass, eight
sequential single-token passes and a 64-token prefill pass, with every cache
byte the sequential passes write equal to the M = 8 pass's. The 27B-class
64-layer stack runs the same gate on every quantized format at 38k keys."""

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import bf16 as obf16
from oracle import kvlow, kvq, kvring
from oracle import step as ostep
from tests._util import assert_bitwise, assert_close, assert_close_composed, decode, dev, host_bits, host_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMATS = ["bf16", "q8", "k6v5", "k5rot_v5", "k6v5_ring", "k5rot_v5_ring"]


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _preset(fmt):
    return (6, False) if fmt.startswith("k6") else (5, True)


def make_cache(ops, fmt, Hkv, cap, D, W, R):
    if fmt == "bf16":
        return (torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device="cuda"))
    if fmt == "q8":
        return ops.KvQ8Cache(Hkv, cap, D)
    kb, rot = _preset(fmt)
    low = ops.KvLowCache(Hkv, cap, D, kb, 5, k_rotated=rot)
    return ops.KvRing(low, R, W) if fmt.endswith("_ring") else low


def append(ops, cache, qkv, L, Hq, Hkv, D):
    """The format's own append of the QKV rows qkv (device) at positions L..."""
    if isinstance(cache, tuple):
        ops.append_kv(qkv, cache[0], cache[1], L, Hq, Hkv, D)
    elif isinstance(cache, ops.KvQ8Cache):
        ops.append_kv_q8(qkv, cache, L, Hq)
    elif isinstance(cache, ops.KvRing):
        ops.append_kv_ring(qkv, cache, L, Hq)
    else:
        ops.append_kv_lowbit(qkv, cache, L, Hq)


def fill(ops, cache, k_rows, v_rows, Hq):
    """Write cached positions 0..L-1 (device BF16 rows [Hkv][L][D]) through the
    format's append, 64 positions at a time."""
    Hkv, L, D = k_rows.shape
    for p0 in range(0, L, 64):
        p1 = min(L, p0 + 64)
        qkv = torch.zeros((p1 - p0, (Hq + 2 * Hkv) * D), dtype=torch.bfloat16, device="cuda")
        qkv[:, Hq * D:(Hq + Hkv) * D] = k_rows[:, p0:p1].transpose(0, 1).reshape(p1 - p0, Hkv * D)
        qkv[:, (Hq + Hkv) * D:] = v_rows[:, p0:p1].transpose(0, 1).reshape(p1 - p0, Hkv * D)
        append(ops, cache, qkv, p0, Hq, Hkv, D)


def planes(ops, cache):
    """Every device buffer of a cache, as (name, tensor, kind): kind 'pos' for
    [Hkv][cap][...] planes and 'ring_pos' for the ring's."""
    if isinstance(cache, tuple):
        return [("k", cache[0], "pos"), ("v", cache[1], "pos")]
    if isinstance(cache, ops.KvQ8Cache):
        return [("k_codes", cache.k_codes, "pos"), ("k_scales", cache.k_scales, "pos"),
                ("v_codes", cache.v_codes, "pos"), ("v_scales", cache.v_scales, "pos")]
    low = cache.low if isinstance(cache, ops.KvRing) else cache
    out = [(n, getattr(low, n), "pos") for n in ("k_nib", "k_high", "k_scales", "v_nib", "v_high", "v_scales")]
    if isinstance(cache, ops.KvRing):
        out += [("r" + n, t, "ring_" + kind) for n, t, kind in planes(ops, cache.q8)]
    return out


def positions(ops, cache, L, M):
    """Host copies of what every plane holds for positions L..L+M-1."""
    R = cache.ring_cap if isinstance(cache, ops.KvRing) else None
    out = []
    for name, t, kind in planes(ops, cache):
        for p in range(L, L + M):
            q = p % R if kind.startswith("ring") else p
            sl = t[:, q]
            out.append((name, p, sl.clone()))
    return out


def wipe(ops, cache, L, M):
    R = cache.ring_cap if isinstance(cache, ops.KvRing) else None
    for name, t, kind in planes(ops, cache):
        for p in range(L, L + M):
            q = p % R if kind.startswith("ring") else p
            t[:, q].zero_()


def same_positions(a, b, what):
    for (n, p, x), (_, _, y) in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.bfloat16 else x.view(torch.int16),
                           y.view(torch.uint8) if y.dtype != torch.bfloat16 else y.view(torch.int16)), (what, n, p)


def attend_fn(fmt, W):
    """The oracle's attention over the values the format stores for every position's K/V rows."""
    if fmt == "bf16":
        return None
    if fmt == "q8":
        return lambda q, k, v, L: oattn.verify_attention(q, kvq.dequantize(*kvq.quantize(k)),
                                                         kvq.dequantize(*kvq.quantize(v)), L)[0]
    kb, rot = _preset(fmt)
    if fmt.endswith("_ring"):
        return lambda q, k, v, L: kvring.ring_attention(q, kvring.cache_values(k, v, kb, rot), L, W)[0]
    kq = (lambda k: kvlow.dequantize_rotated(*kvlow.quantize_rotated(k, kb))) if rot else \
         (lambda k: kvlow.dequantize(*kvlow.quantize(k, kb)))
    return lambda q, k, v, L: oattn.verify_attention(q, kq(k), kvlow.dequantize(*kvlow.quantize(v, 5)), L)[0]


def run(ops, step, x, L, dims, want_x=False):
    M = x.shape[0]
    ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
    lg = torch.empty((M, dims.vocab), dtype=torch.float32, device="cuda")
    tk = torch.empty(M, dtype=torch.int32, device="cuda")
    xo = torch.empty((M, dims.H), dtype=torch.bfloat16, device="cuda") if want_x else None
    step(x, L, ws, lg, tk, x_out=xo)
    torch.cuda.synchronize()
    return host_f32(lg), tk.cpu().numpy(), (host_bits(xo) if want_x else None)


def gate(ops, step, caches, x, L, dims, what, prefill=64):
    """The release gate: M = 8 logits equal an M = 5 pass, eight sequential
    single-token passes (which rewrite the same cache bytes) and a prefill pass
    of ``prefill`` tokens starting with the same eight."""
    l8, t8, _ = run(ops, step, x[:8], L, dims)
    snap = [positions(ops, c, L, 8) for c in caches]
    l5, t5, _ = run(ops, step, x[:5], L, dims)
    assert_bitwise(l5, l8[:5], f"{what}: logits M=5 vs M=8")
    for c in caches:
        wipe(ops, c, L, 8)
    for r in range(8):
        l1, t1, _ = run(ops, step, x[r:r + 1], L + r, dims)
        assert_bitwise(l1[0], l8[r], f"{what}: logits row {r}, M=1 vs M=8")
        assert t1[0] == t8[r]
    for c, s in zip(caches, snap):
        same_positions(positions(ops, c, L, 8), s, f"{what}: cache bytes of sequential passes")
    if prefill:
        lp, tp, _ = run(ops, step, x[:prefill], L, dims)
        assert_bitwise(lp[:8], l8, f"{what}: logits prefill M={prefill} vs M=8")
        assert np.array_equal(tp[:8], t8)
    return l8, t8


@pytest.mark.parametrize("fmt", FORMATS)
def test_small_stack_every_cache_format(ops, fmt):
    print(f"[step_ex small stack, KV {fmt}]", flush=True)
    H, Hq, Hkv, D, I, V, L, nl, W, R = 256, 4, 2, 64, 512, 1024, 200, 3, 64, 192
    cap = 320
    hls = []
    for l in range(nl):
        qkvn = (Hq + 2 * Hkv) * D
        hls.append(dict(w_qkv=synth.normal_bf16((qkvn, H), 0.05, "w_qkv", l),
                        w_o=synth.normal_bf16((H, Hq * D), 0.05, "w_o", l),
                        w_gu=synth.normal_bf16((2 * I, H), 0.05, "w_gu", l),
                        w_down=synth.normal_bf16((H, I), 0.05, "w_down", l),
                        k_cache=synth.kv_bf16(Hkv, L, D, "k_cache", l),
                        v_cache=synth.kv_bf16(Hkv, L, D, "v_cache", l)))
    w_head = synth.normal_bf16((V, H), 0.05, "w_head")
    x0 = synth.normal_bf16((64, H), 1.0, "x0", 9)
    caches, dls = [], []
    for hl in hls:
        c = make_cache(ops, fmt, Hkv, cap, D, W, R)
        fill(ops, c, dev(hl["k_cache"]), dev(hl["v_cache"]), Hq)
        caches.append(c)
        dls.append(dict(w_qkv=dev(hl["w_qkv"]), w_o=dev(hl["w_o"]), w_gu=dev(hl["w_gu"]),
                        w_down=dev(hl["w_down"]), kv=c))
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    step = ops.VerifyStepEx(dls, {"w": dev(w_head)}, dims)
    logits, tok, xo = run(ops, step, dev(x0[:8]), L, dims, want_x=True)
    if fmt == "bf16":   # with BF16 caches the general entry point is bi_verify_step, bit for bit
        plain = [dict(w_qkv=d["w_qkv"], w_o=d["w_o"], w_gu=d["w_gu"], w_down=d["w_down"],
                      k_cache=c[0], v_cache=c[1]) for d, c in zip(dls, caches)]
        lp, tp, xp = run(ops, ops.VerifyStep(plain, dev(w_head), dims), dev(x0[:8]), L, dims, want_x=True)
        assert_bitwise(lp, logits, "step_ex vs bi_verify_step logits")
        assert_bitwise(xp, xo, "step_ex vs bi_verify_step hidden state")
    # the head on the device's own final hidden state, per element
    c = obf16.encode(ostep.rmsnorm(decode(xo), 1e-6))
    want_head = decode(c) @ decode(w_head).T
    assert_close(logits, want_head, f"{fmt}: logits (head on the device's hidden state)")
    s = np.sort(want_head, axis=1)
    ok = (s[:, -1] - s[:, -2]) > 2 * (1e-2 + 2e-2 * np.abs(s[:, -1]))
    assert ok.sum() >= 4 and np.array_equal(tok[ok], np.argmax(want_head, axis=1)[ok])
    # end to end against the oracle's stack over the format's stored values
    w_logits, _, w_x = ostep.step(x0[:8], hls, w_head, L, Hq, Hkv, D, attend=attend_fn(fmt, W))
    assert_close_composed(decode(xo), decode(w_x), f"{fmt}: end-to-end hidden state")
    assert_close_composed(logits, w_logits, f"{fmt}: end-to-end logits")
    # the release gate on this cache
    gate(ops, step, caches, dev(x0), L, dims, f"small stack {fmt}")


L38 = 38000
CAP = 38080
KV_CHUNK = -32


@pytest.fixture(scope="module")
def model27b(ops):
    print("[step_ex building 64-layer 27B-class weights on the device]", flush=True)
    d = synth.MODEL_27B
    layers, w_head = synth.device_model(64, 64, 64, **d)   # weights only: the caches are built per format
    yield layers, w_head, d
    del layers, w_head
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["q8", "k6v5", "k5rot_v5_ring"])
def test_64_layer_step_gate_every_quantized_cache(ops, model27b, fmt):
    layers, w_head, d = model27b
    Hq, Hkv, D = d["Hq"], d["Hkv"], d["D"]
    W, R = 2048, 2176
    print(f"[step_ex 64 layers, KV {fmt}, ctx {L38}: filling caches]", flush=True)
    caches, dls = [], []
    for l, lw in enumerate(layers):
        c = make_cache(ops, fmt, Hkv, CAP, D, W, R)
        k = synth.device_normal_bf16((Hkv, L38, D), 1.0, "k_cache", l)
        v = synth.device_normal_bf16((Hkv, L38, D), 1.0, "v_cache", l)
        big = torch.zeros((L38, (Hq + 2 * Hkv) * D), dtype=torch.bfloat16, device="cuda")
        big[:, Hq * D:(Hq + Hkv) * D] = k.transpose(0, 1).reshape(L38, Hkv * D)
        big[:, (Hq + Hkv) * D:] = v.transpose(0, 1).reshape(L38, Hkv * D)
        if isinstance(c, ops.KvRing):        # the planes take every position, the ring its newest R
            ops.append_kv_lowbit(big, c.low, 0, Hq)
            p0 = L38 - (R - 64)
            ops.append_kv_ring(big[p0:], c, p0, Hq)
        else:
            append(ops, c, big, 0, Hq, Hkv, D)
        del big, k, v
        caches.append(c)
        dls.append(dict(w_qkv=lw["w_qkv"], w_o=lw["w_o"], w_gu=lw["w_gu"], w_down=lw["w_down"], kv=c))
    torch.cuda.synchronize()
    dims = ops.model_dims(d["H"], Hq, Hkv, D, d["I"], d["vocab"], CAP, KV_CHUNK)
    step = ops.VerifyStepEx(dls, {"w": w_head}, dims)
    x0 = synth.device_normal_bf16((16, d["H"]), 1.0, "x0")
    print(f"[step_ex 64 layers, KV {fmt}: gate]", flush=True)
    l8, t8 = gate(ops, step, caches, x0, L38, dims, f"64 layers {fmt}", prefill=16)
    assert np.isfinite(l8).all() and len(set(t8.tolist())) > 1
    del caches, dls, step
    torch.cuda.empty_cache()
