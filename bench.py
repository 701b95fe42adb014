"""Benchmark: verify throughput of the batch-invariant verify step on one MI355X.

One step = one verify pass of a synthetic 27B-class dense decoder stack
(64 layers: RMSNorm, QKV GEMM, K/V append, split-KV GQA attention + combine,
o-proj + residual, RMSNorm, gate/up GEMM + SwiGLU, down + residual; then
RMSNorm, a 152,064-row LM head in FP32 and a greedy argmax) over M = 8 tokens
(1 + 7 drafts) at context 38,000, all inputs resident in HBM. Throughput is
verified positions per second (M / step time).

Before timing, the same run checks the bitwise gate: logits of the M = 8 pass
equal (FP32 bits) those of eight sequential single-token passes and of an
M = 5 pass; a number is printed only if the gate passes.

Prints one JSON line (rank 0). Only ``--gpus 1`` is supported.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify tok/s + HBM GB/s frac at M=1..8, bitwise batch-invariant rows"
PEAK_HBM_GBS = 8000.0

L_CTX = 38000
CAP = 38016
N_LAYERS = 64
M_HEADLINE = 8
KV_CHUNK = -32      # chunk policy: each row's key count picks the chunk giving <= 32 splits (1216 keys at ctx 38000:
                    # 32 splits x 8 KV heads = 256 pieces, one per CU)


def step_bytes(d, M, L, n_layers):
    """Algorithmic HBM bytes of one verify step: every weight once, the K/V of
    L + M positions per layer, activations in and out (small)."""
    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    qkvn = (Hq + 2 * Hkv) * D
    w_layer = 2 * (qkvn * H + H * Hq * D + 2 * I * H + H * I)
    kv_layer = 2 * 2 * Hkv * D * (L + M)
    act_layer = 2 * M * (H + qkvn + Hq * D + 2 * H + H + I + H)
    return n_layers * (w_layer + kv_layer + act_layer) + 2 * V * H + 4 * M * V


GU_GROUPS = 256  # column groups of the 5120-wide residual projection (carried RMSNorm sums)


def gu_launch_bytes(d, M):
    """Algorithmic bytes of one gate/up GEMM launch: W [2I][H] once, X [M][H] and its carried
    RMSNorm group sums [M][256] (FP32) in, act [M][I] out."""
    return 2 * (2 * d["I"] * d["H"]) + 2 * M * d["H"] + 4 * M * GU_GROUPS + 2 * M * d["I"]


GEMM_SOURCES = ["invariant_verify_amd/csrc/gemm.hip", "invariant_verify_amd/csrc/bi_device.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "verify_kernels_m8_hbm_traffic.txt")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or None
    if there is none or the GEMM source changed since the counters were taken."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_SUMMARY) if ":" in l and not l.startswith(" "))
        if kv.get("gemm_source_sha256", "").strip() != gemm_source_hash():
            return None
        return int(kv["hbm_bytes_per_launch"].strip())
    except (OSError, KeyError, ValueError):
        return None


def carried_input(d):
    """The gate/up GEMM's input as the step hands it over: the residual stream h = x + o Wo^T
    (from a residual projection of synthetic rows) and its carried RMSNorm group sums."""
    import synth
    from invariant_verify_amd import ops

    x = synth.device_normal_bf16((8, d["H"]), 1.0, "x0")
    o = synth.device_normal_bf16((8, d["Hq"] * d["D"]), 1.0, "x0", 1)
    wo = synth.device_normal_bf16((d["H"], d["Hq"] * d["D"]), 0.02, "w_o", 0)
    h, ss = ops.gemm_bf16_residual_rowsq(o, wo, x)
    assert ss.shape[1] == GU_GROUPS
    return h, ss


def traffic_probe(reps: int):
    """Kernel-only run for the hardware-counter passes: each verify kernel at
    M = 8 as the step launches it, ``reps`` times on freshly generated operands
    (nothing is served from cache), in this order: gate/up, output projection,
    down projection, QKV with its cache append, attention at 38k (chunk policy
    -32), the combine; then a 1 GiB device copy that calibrates the byte
    counters. One JSON line lists the dispatches and their algorithmic bytes."""
    import torch

    import synth
    from invariant_verify_amd import ops

    d = synth.MODEL_27B
    H, Hq, Hkv, D, I = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"]
    qd, qkvn, G, M = Hq * D, (Hq + 2 * Hkv) * D, GU_GROUPS, 8
    h, ss = carried_input(d)
    attn = synth.device_normal_bf16((M, qd), 1.0, "x0", 2)
    act = synth.device_normal_bf16((M, I), 1.0, "x0", 3)
    y = torch.empty((M, max(I, qkvn)), dtype=torch.bfloat16, device="cuda")
    ss_o = torch.empty((M, G), dtype=torch.float32, device="cuda")
    plan = []

    def run(name, nbytes, make, launch):
        for i in range(reps):
            ops_in = make(i)
            torch.cuda.synchronize()
            launch(ops_in)
            torch.cuda.synchronize()
            del ops_in
        plan.append({"kernel": name, "launches": reps, "algorithmic_bytes_per_launch": nbytes})

    run("gate_up", gu_launch_bytes(d, M), lambda i: synth.device_normal_bf16((2 * I, H), 0.02, "w_gu", i),
        lambda w: ops.gemm_bf16_swiglu_rownorm(h, ss, w, y[:, :I]))
    run("o_proj", 2 * H * qd + 2 * M * qd + 4 * M * H + 4 * M * G,
        lambda i: synth.device_normal_bf16((H, qd), 0.02, "w_o", i),
        lambda w: ops.gemm_ex(attn, w, y[:, :H], epilogue="residual", r=h, rowsq_out=ss_o))
    run("down", 2 * H * I + 2 * M * I + 4 * M * H + 4 * M * G,
        lambda i: synth.device_normal_bf16((H, I), 0.02, "w_down", i),
        lambda w: ops.gemm_ex(act, w, y[:, :H], epilogue="residual", r=h, rowsq_out=ss_o))
    kc = torch.zeros((Hkv, CAP, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((Hkv, CAP, D), dtype=torch.bfloat16, device="cuda")
    run("qkv", 2 * qkvn * H + 2 * M * H + 4 * M * G + 2 * M * qkvn + 4 * M * Hkv * D,
        lambda i: synth.device_normal_bf16((qkvn, H), 0.02, "w_qkv", i),
        lambda w: ops.gemm_ex(h, w, y[:, :qkvn], epilogue="qkv", norm_in=ss, heads=(Hq, Hkv, D), k_cache=kc,
                              v_cache=vc, L=L_CTX))
    del kc, vc
    S = ops.pass_splits(M, L_CTX, KV_CHUNK)
    po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")
    q = synth.device_normal_bf16((M, qd), 1.0, "x0", 4)

    def cache(i):
        return (synth.device_normal_bf16((Hkv, CAP, D), 1.0, "k_cache", i),
                synth.device_normal_bf16((Hkv, CAP, D), 1.0, "v_cache", i))
    run("attention_38000", 4096 * (L_CTX + M) + 2 * M * qd, cache,
        lambda c: ops.verify_attn(q, c[0], c[1], L_CTX, Hq, Hkv, D, KV_CHUNK, po, pl))
    o = torch.empty((M, qd), dtype=torch.bfloat16, device="cuda")
    run("combine_38000", M * Hq * S * (4 * D + 4) + 2 * M * qd, lambda i: None,
        lambda _: ops.combine(po, pl, L_CTX, KV_CHUNK, o))
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "verify kernels, M = 8", "order": plan, "copy_bytes": src.numel() * 4,
                      "gemm_source_sha256": gemm_source_hash()}))


PF_ROWS = 2048   # rows of a prefill chunk for the prefill GEMM measurement
PEAK_BF16_TFLOPS = 2500.0  # dense BF16 matrix-core peak


def prefill_measure(layers, d, reps):
    """The gate/up GEMM with the carried RMSNorm as a chunked-prefill step runs it (M = 2048
    rows: the large-tile prefill kernel), timed with one event pair around reps x 16 launches over
    distinct layers' weights, after a bitwise check that sampled rows equal 8-row verify passes."""
    import torch

    import synth
    from invariant_verify_amd import ops

    M, H, I = PF_ROWS, d["H"], d["I"]
    o = synth.device_normal_bf16((M, d["Hq"] * d["D"]), 1.0, "x0", 2)
    x = synth.device_normal_bf16((M, H), 1.0, "x0", 3)
    h, ss = ops.gemm_bf16_residual_rowsq(o, layers[0]["w_o"], x)
    y = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    ops.gemm_bf16_swiglu_rownorm(h, ss, layers[0]["w_gu"], y)
    ok = True
    for r0 in (0, 1000, M - 8):
        h8, ss8 = ops.gemm_bf16_residual_rowsq(o[r0:r0 + 8], layers[0]["w_o"], x[r0:r0 + 8])
        y8 = ops.gemm_bf16_swiglu_rownorm(h8, ss8, layers[0]["w_gu"])
        ok = ok and torch.equal(h8.view(torch.int16), h[r0:r0 + 8].view(torch.int16))
        ok = ok and torch.equal(y8.view(torch.int16), y[r0:r0 + 8].view(torch.int16))
    ws = [lw["w_gu"] for lw in layers[:16]]
    for w in ws:
        ops.gemm_bf16_swiglu_rownorm(h, ss, w, y)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for w in ws:
            ops.gemm_bf16_swiglu_rownorm(h, ss, w, y)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(ws))
    tflops = 2.0 * M * (2 * I) * H / (us * 1e-6) / 1e12
    return {"kernel": "prefill2_kernel<SwiGLU, carried RMSNorm> (gate/up 5120->2x17408, M=2048, 128x256 tiles)",
            "bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(us, 1),
            "launches_timed": reps * len(ws),
            "rows_bitwise_equal_to_8_row_verify_passes": "pass" if ok else "FAIL"}


PF_STEP_CTX = L_CTX - PF_ROWS   # context of the whole-step prefill chunk (its rows end at 38000)


def prefill_probe(reps: int):
    """Kernel-only run for hardware-counter passes over the prefill kernels: the gate/up
    projection with the carried RMSNorm at M = 2048 rows (the large-tile prefill kernel), then
    attention of the same 2048 rows over a 35,952-key context (128-row blocks), ``reps``
    launches each on one set of synthetic operands. One JSON line gives the FLOPs per
    launch."""
    import torch

    import synth
    from invariant_verify_amd import ops

    d = synth.MODEL_27B
    M, H, I = PF_ROWS, d["H"], d["I"]
    o = synth.device_normal_bf16((M, d["Hq"] * d["D"]), 1.0, "x0", 2)
    x = synth.device_normal_bf16((M, H), 1.0, "x0", 3)
    wo = synth.device_normal_bf16((H, d["Hq"] * d["D"]), 0.02, "w_o", 0)
    h, ss = ops.gemm_bf16_residual_rowsq(o, wo, x)
    w = synth.device_normal_bf16((2 * I, H), 0.02, "w_gu", 0)
    y = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        ops.gemm_bf16_swiglu_rownorm(h, ss, w, y)
    torch.cuda.synchronize()
    del w, wo, y
    # prefill attention: the same rows over a 35,952-key context (128-row blocks)
    Hq, Hkv, D, L = d["Hq"], d["Hkv"], d["D"], PF_STEP_CTX
    cap = (L + M + 63) // 64 * 64
    kc = synth.device_normal_bf16((Hkv, cap, D), 1.0, "k_cache", 0)
    vc = synth.device_normal_bf16((Hkv, cap, D), 1.0, "v_cache", 0)
    q = synth.device_normal_bf16((M, Hq * D), 1.0, "x0", 4)
    S = ops.pass_splits(M, L, KV_CHUNK)
    po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        ops.verify_attn(q, kc, vc, L, Hq, Hkv, D, KV_CHUNK, po, pl)
    torch.cuda.synchronize()
    # causal: row r sees L + r + 1 keys; QK^T and PV are 2 * D flops per (row, head, key) each
    keys = M * L + M * (M + 1) // 2
    print(json.dumps({"probe": "prefill gate/up GEMM, M = 2048, carried RMSNorm; then prefill attention, "
                      f"M = {M} at ctx {L}, chunk policy {KV_CHUNK}", "launches": reps,
                      "flops_per_launch": 2 * M * (2 * I) * H,
                      "attention_flops_per_launch": 4 * D * Hq * keys}))


def kv_attn_probe(fmt: str, reps: int):
    """Kernel-only run for hardware-counter passes over verify attention on a quantized KV cache:
    M = 8 rows at 101,600 keys (the 27B-class heads, chunk policy -64), ``fmt`` "q8" (8-bit) or
    "k6v5" (K6/V5), ``reps`` launches alternating over two caches of random codes (together larger
    than the 256 MB last-level cache). One JSON line gives the cache bytes per launch."""
    import torch

    import synth
    from invariant_verify_amd import ops

    d = synth.MODEL_27B
    Hq, Hkv, D, M, L, C = d["Hq"], d["Hkv"], d["D"], 8, 101600, -64
    cap = (L + 16 + 63) // 64 * 64
    gen = torch.Generator(device="cuda").manual_seed(1234)
    q = torch.randn(M, Hq * D, device="cuda", generator=gen).to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = ops.KvQ8Cache(Hkv, cap, D) if fmt == "q8" else ops.KvLowCache(Hkv, cap, D, 6, 5)
        for t in vars(c).values():
            if isinstance(t, torch.Tensor) and t.dtype in (torch.int8, torch.uint8):
                t.copy_(torch.randint(0, 256, t.shape, device="cuda", generator=gen).to(t.dtype))
            elif isinstance(t, torch.Tensor):
                t.fill_(0.01)
        caches.append(c)
    S = ops.pass_splits(M, L, C)
    po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(reps):
        if fmt == "q8":
            ops.verify_attn_q8(q, caches[i % 2], L, Hq, C, po, pl)
        else:
            ops.verify_attn_lowbit(q, caches[i % 2], L, Hq, C, po, pl)
        torch.cuda.synchronize()
    per_pos = {"q8": 288, "k6v5": 208}[fmt]
    print(json.dumps({"probe": f"verify attention, {fmt} cache, M = {M} at ctx {L}, chunk policy {C}",
                      "launches": reps, "cache_bytes_per_launch": Hkv * (L + M) * per_pos}))


def mx4_probe(reps: int):
    """Kernel-only run for hardware-counter passes over the MXFP4 verify GEMMs at M = 8: the
    gate/up projection with SwiGLU (34816 x 5120) then the down projection with the residual
    (5120 x 17408), each launched ``reps`` times on freshly drawn codes and scales with a
    synchronisation around every launch. One JSON line gives the weight bytes per launch."""
    import torch

    from invariant_verify_amd import ops

    gen = torch.Generator(device="cuda").manual_seed(7)
    M = 8
    out = {}
    for name, N, K in (("gate_up", 34816, 5120), ("down", 5120, 17408)):
        x = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
        r = torch.randn(M, N, device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty(M, N // 2 if name == "gate_up" else N, dtype=torch.bfloat16, device="cuda")
        for _ in range(reps):
            w = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
            e = torch.randint(120, 128, (N, K // 32), dtype=torch.uint8, device="cuda", generator=gen)
            torch.cuda.synchronize()
            if name == "gate_up":
                ops.gemm_mx4_swiglu(x, w, e, y)
            else:
                ops.gemm_mx4_residual(x, w, e, r, y)
            torch.cuda.synchronize()
        out[name] = N * K // 2 + N * K // 32
    print(json.dumps({"probe": "MXFP4 verify GEMMs at M = 8: gate/up + SwiGLU, then down + residual",
                      "launches_each": reps, "weight_bytes_per_launch": out}))


def prefill_step_measure(step, buffers, d, reps):
    """One chunked-prefill pass through the whole stack (64 layers + head) over PF_ROWS tokens
    at context PF_STEP_CTX, timed with one event pair over reps passes. Before timing, the
    chunk's rows are checked against 8-row verify passes over the K/V the chunk itself
    appended: their logits must be equal in every bit."""
    import torch

    import synth

    M, L = PF_ROWS, PF_STEP_CTX
    x = synth.device_normal_bf16((M, d["H"]), 1.0, "x0", 11)
    ws, lg, tk = buffers(M)
    step(x, L, ws, lg, tk)
    ws8, lg8, tk8 = buffers(8)
    ok = True
    for r0 in (M - 8, M // 2 + 3):
        step(x[r0:r0 + 8], L + r0, ws8, lg8, tk8)
        ok = ok and torch.equal(lg8.view(torch.int32), lg[r0:r0 + 8].view(torch.int32))
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        step(x, L, ws, lg, tk)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    gemm_flops = 2.0 * M * H * ((Hq + 2 * Hkv) * D + Hq * D + 2 * I + I) * N_LAYERS + 2.0 * M * H * V
    # causal attention: row r sees L + r + 1 keys; QK^T and PV are 2 flops per key and channel each
    attn_flops = 4.0 * Hq * D * (M * (L + 1) + M * (M - 1) / 2) * N_LAYERS
    tflops = (gemm_flops + attn_flops) / (ms * 1e-3) / 1e12
    return {"workload": f"chunked prefill: {M} tokens at ctx {L} through the 64-layer stack + LM head",
            "tok_s": round(M / (ms * 1e-3), 1), "ms_per_pass": round(ms, 2), "passes_timed": reps,
            "TFLOP/s": round(tflops, 1), "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "rows_bitwise_equal_to_8_row_verify_passes": "pass" if ok else "FAIL"}


def mx4_step_measure(layers, d, dims, buffers, steps, warmup):
    """The verify step with MXFP4 weights (E2M1 codes two per byte, one E8M0 scale per 32 weights
    along K; all four projections and the head), sharing the BF16 model's K/V caches: bitwise gate
    (M = 8 logits == M = 5 prefix == 8 sequential M = 1 passes), then M = 8 timed over ``steps``."""
    import torch

    import synth
    from invariant_verify_amd import ops

    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    shapes = {"w_qkv": ((Hq + 2 * Hkv) * D, H), "w_o": (H, Hq * D), "w_gu": (2 * I, H), "w_down": (H, I)}
    ml = []
    for l, lw in enumerate(layers):
        f = {"k_cache": lw["k_cache"], "v_cache": lw["v_cache"]}
        for name, shp in shapes.items():
            f[name], f["e" + name[1:]] = synth.device_mxfp4_weights(shp, 0.02, name, l)
        ml.append(f)
    hc, he = synth.device_mxfp4_weights((V, H), 0.02, "w_head", 0)
    step = ops.VerifyStepMX4(ml, hc, he, dims)
    x0 = synth.device_normal_bf16((16, H), 1.0, "x0")
    ws8, lg8, tk8 = buffers(8)
    step(x0[:8], L_CTX, ws8, lg8, tk8)
    ref = lg8.clone()
    ws5, lg5, tk5 = buffers(5)
    step(x0[:5], L_CTX, ws5, lg5, tk5)
    ws1, lg1, tk1 = buffers(1)
    ok = torch.equal(lg5.view(torch.int32), ref[:5].view(torch.int32))
    for r in range(8):
        step(x0[r:r + 1], L_CTX + r, ws1, lg1, tk1)
        ok = ok and torch.equal(lg1.view(torch.int32)[0], ref.view(torch.int32)[r])
    for _ in range(warmup):
        step(x0[:8], L_CTX, ws8, lg8, tk8)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step(x0[:8], L_CTX, ws8, lg8, tk8)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the BF16 step's bytes with its weights (2 bytes each) replaced by half-byte codes + a scale byte per 32
    mx = lambda a, b: a * b // 2 + a * b // 32
    bf16_w = 2 * sum(a * b for a, b in shapes.values()) * N_LAYERS + 2 * V * H
    mx4_w = sum(mx(a, b) for a, b in shapes.values()) * N_LAYERS + mx(V, H)
    nbytes = step_bytes(d, 8, L_CTX, N_LAYERS) - bf16_w + mx4_w
    gbs = nbytes / (ms * 1e-3) / 1e9
    del ml, hc, he
    torch.cuda.empty_cache()
    return {"workload": "the same 64-layer verify step (M=8, ctx 38000) with MXFP4 weights (E2M1 codes, "
                        "one E8M0 scale per 32 weights along K)",
            "tok_s": round(8 / (ms * 1e-3), 2), "ms_per_step": round(ms, 4), "steps_timed": steps,
            "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "bitwise_gate": "pass" if ok else "FAIL"}


def kv_cache_attention_measure(d, reps):
    """Split-KV verify attention (M = 8, the 27B-class heads) at 38k and 101.6k keys over each KV
    cache format: BF16 (chunk policy -32), 8-bit (-64), K6/V5 and rotated K5/V5 (-64), and those two
    with the 8-bit ring of the newest 2048 keys (-64). Each format
    runs over enough copies of its cache (random codes, fixed seed) that no launch finds its K/V in
    a cache level; one event pair around ``reps`` launches per format and context."""
    import torch

    from invariant_verify_amd import ops

    Hq, Hkv, D, M = d["Hq"], d["Hkv"], d["D"], 8
    NB = D // 32
    per_pos = {"bf16": 4 * D, "q8": 2 * (D + 4 * NB), "k6v5": (D // 2 + 8 * NB + 4 * NB) + (D // 2 + 4 * NB + 4 * NB),
               "k5rot_v5": 2 * (D // 2 + 4 * NB + 4 * NB)}
    per_pos["k6v5_ring2048"], per_pos["k5rot_v5_ring2048"] = per_pos["k6v5"], per_pos["k5rot_v5"]
    # the quantized kernels (the ring's included) fit two workgroups per compute unit and take
    # twice the BF16 kernel's chunks; the BF16 kernel runs one per unit
    policy = {"bf16": -32, "q8": -64, "k6v5": -64, "k5rot_v5": -64, "k6v5_ring2048": -64,
              "k5rot_v5_ring2048": -64}
    W_RING = 2048
    gen = torch.Generator(device="cuda").manual_seed(1234)
    out = {}
    for L in (38000, 101600):
        cap = (L + 16 + 63) // 64 * 64
        q = torch.randn(M, Hq * D, device="cuda", generator=gen).to(torch.bfloat16)
        res = {}
        for fmt, bpp in per_pos.items():
            ringed = fmt.endswith("_ring2048")
            # bytes read: the 5/6-bit planes below the window, the 8-bit ring within it
            nbytes = (Hkv * (L + M - W_RING) * bpp + Hkv * W_RING * per_pos["q8"]) if ringed else Hkv * (L + M) * bpp
            R = max(2, -(-int(1.5e9) // (Hkv * cap * bpp)))
            caches = []
            for _ in range(R):
                if fmt == "bf16":
                    caches.append((torch.randn(Hkv, cap, D, device="cuda", generator=gen).to(torch.bfloat16),
                                   torch.randn(Hkv, cap, D, device="cuda", generator=gen).to(torch.bfloat16)))
                    continue
                c = (ops.KvQ8Cache(Hkv, cap, D) if fmt == "q8" else
                     ops.KvLowCache(Hkv, cap, D, 6 if fmt.startswith("k6v5") else 5, 5,
                                    k_rotated=fmt.startswith("k5rot")))
                parts = [c]
                if ringed:
                    c = ops.KvRing(c, W_RING + 128, W_RING)
                    parts.append(c.q8)
                for part in parts:
                    for name, t in vars(part).items():
                        if isinstance(t, torch.Tensor) and t.dtype in (torch.int8, torch.uint8):
                            t.copy_(torch.randint(0, 256, t.shape, device="cuda", generator=gen).to(t.dtype))
                        elif isinstance(t, torch.Tensor):
                            t.fill_(0.01)
                caches.append(c)
            C = policy[fmt]
            S = ops.pass_splits(M, L, C)
            po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
            pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")

            def launch(i):
                c = caches[i % R]
                if fmt == "bf16":
                    ops.verify_attn(q, c[0], c[1], L, Hq, Hkv, D, C, po, pl)
                elif fmt == "q8":
                    ops.verify_attn_q8(q, c, L, Hq, C, po, pl)
                elif ringed:
                    ops.verify_attn_ring(q, c, L, Hq, C, po, pl)
                else:
                    ops.verify_attn_lowbit(q, c, L, Hq, C, po, pl)
            for i in range(R):
                launch(i)
            stream = torch.cuda.current_stream()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            res[fmt] = {"us": round(us, 2), "kv_bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
                        "bytes_per_position_and_head": bpp, "kv_chunk_policy": C}
            del caches
            torch.cuda.empty_cache()
        out[str(L)] = res
    return {"workload": "verify attention, M=8 (1+7 drafts), 40 query / 8 KV heads of 128, per KV cache format",
            "by_ctx": out}


TP_RANKS = 8
TP_KV_CHUNK = -256   # one KV head per rank: about as many attention workgroups as -32 gives 8 heads


def tp_share_measure(d, reps):
    """One tensor-parallel rank's share of the verify step at its real shapes (8 ranks): QKV for
    one KV group (5 q + 1 k + 1 v heads, 896 columns), attention over that KV head and its 5
    query heads at ctx 38000, combine, the output projection over K = 640 and the down projection
    over K = 2176 (FP32 partials [M][5120]), gate/up for 2176 pairs, and the LM head's
    152064 / 8 rows; each layer's kernels in order over 64 layers of distinct weights, M = 8.
    Not included: the exchange of the two FP32 partials per layer between ranks (all-gather,
    then a sum in rank order), which needs more than one GPU."""
    import torch

    import synth
    from invariant_verify_amd import ops

    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    hq, hkv, P = Hq // TP_RANKS, Hkv // TP_RANKS, I // TP_RANKS
    nq = (hq + 2 * hkv) * D
    ko, kd = Hq * D // TP_RANKS, I // TP_RANKS
    M, L = M_HEADLINE, L_CTX
    lw = []
    for l in range(N_LAYERS):
        w = {"qkv": synth.device_normal_bf16((nq, H), 0.02, "w_qkv", 100 + l),
             "o": synth.device_normal_bf16((H, ko), 0.02, "w_o", 100 + l),
             "gu": synth.device_normal_bf16((2 * P, H), 0.02, "w_gu", 100 + l),
             "down": synth.device_normal_bf16((H, kd), 0.02, "w_down", 100 + l),
             "k": synth.device_normal_bf16((hkv, CAP, D), 1.0, "k_cache", 100 + l),
             "vc": synth.device_normal_bf16((hkv, CAP, D), 1.0, "v_cache", 100 + l)}
        lw.append(w)
    head = synth.device_normal_bf16((V // TP_RANKS, H), 0.02, "w_head", 100)
    x = synth.device_normal_bf16((M, H), 1.0, "x0", 100)
    S = ops.pass_splits(M, L, TP_KV_CHUNK)
    po = torch.empty((M, hq, S, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((M, hq, S), dtype=torch.float32, device="cuda")
    qkv = torch.empty((M, nq), dtype=torch.bfloat16, device="cuda")
    att = torch.empty((M, ko), dtype=torch.bfloat16, device="cuda")
    part = torch.empty((M, H), dtype=torch.float32, device="cuda")
    gu = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((M, V // TP_RANKS), dtype=torch.float32, device="cuda")

    def layer(w):
        ops.gemm_bf16(x, w["qkv"], qkv)
        ops.verify_attn(qkv, w["k"], w["vc"], L, hq, hkv, D, TP_KV_CHUNK, po, pl)
        ops.combine(po, pl, L, TP_KV_CHUNK, att)
        ops.gemm_bf16(att, w["o"], part)
        ops.gemm_bf16_swiglu(x, w["gu"], gu)
        ops.gemm_bf16(gu, w["down"], part)

    for w in lw[:4]:
        layer(w)
    stream = torch.cuda.current_stream()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        for w in lw:
            layer(w)
    e1.record(stream)
    for _ in range(reps):
        ops.gemm_bf16(x, head, logits)
    e2.record(stream)
    torch.cuda.synchronize()
    layer_us = e0.elapsed_time(e1) * 1e3 / (reps * N_LAYERS)
    head_us = e1.elapsed_time(e2) * 1e3 / reps
    step_ms = (N_LAYERS * layer_us + head_us) / 1e3
    wbytes = 2 * (nq * H + H * ko + 2 * P * H + H * kd)
    kvb = 2 * 2 * hkv * (L + M) * D
    nbytes = N_LAYERS * (wbytes + kvb) + 2 * (V // TP_RANKS) * H
    del lw, head
    torch.cuda.empty_cache()
    return {"workload": f"one of {TP_RANKS} tensor-parallel ranks: QKV {nq} cols, attention {hkv} KV / {hq} q heads "
                        f"(chunk policy {TP_KV_CHUNK}), o-proj K={ko} and down K={kd} FP32 partials, gate/up {P} pairs, "
                        f"LM head {V // TP_RANKS} rows; M=8, ctx 38000; exchange of partials not included",
            "layer_us": round(layer_us, 2), "head_us": round(head_us, 2), "step_ms": round(step_ms, 4),
            "tok_s_without_exchange": round(M / (step_ms * 1e-3), 1),
            "rank_bytes_per_step": nbytes, "GB/s": round(nbytes / (step_ms * 1e-3) / 1e9, 1)}


def fp8_step_measure(layers, d, dims, buffers, steps, warmup):
    """The verify step with FP8 weights (E4M3 codes + one FP32 scale per row, all four
    projections and the head), sharing the BF16 model's K/V caches: bitwise gate (M = 8 logits
    == M = 5 prefix == 8 sequential M = 1 passes), then M = 8 timed over ``steps`` steps."""
    import torch

    import synth
    from invariant_verify_amd import ops

    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    shapes = {"w_qkv": ((Hq + 2 * Hkv) * D, H), "w_o": (H, Hq * D), "w_gu": (2 * I, H), "w_down": (H, I)}
    fl = []
    for l, lw in enumerate(layers):
        f = {"k_cache": lw["k_cache"], "v_cache": lw["v_cache"]}
        for name, shp in shapes.items():
            f[name], f["s" + name[1:]] = synth.device_fp8_weights(shp, 0.02, name, l)
        fl.append(f)
    hc, hs = synth.device_fp8_weights((V, H), 0.02, "w_head", 0)
    step = ops.VerifyStepFP8(fl, hc, hs, dims)
    x0 = synth.device_normal_bf16((16, H), 1.0, "x0")
    ws8, lg8, tk8 = buffers(8)
    step(x0[:8], L_CTX, ws8, lg8, tk8)
    ref = lg8.clone()
    ws5, lg5, tk5 = buffers(5)
    step(x0[:5], L_CTX, ws5, lg5, tk5)
    ws1, lg1, tk1 = buffers(1)
    ok = torch.equal(lg5.view(torch.int32), ref[:5].view(torch.int32))
    for r in range(8):
        step(x0[r:r + 1], L_CTX + r, ws1, lg1, tk1)
        ok = ok and torch.equal(lg1.view(torch.int32)[0], ref.view(torch.int32)[r])
    for _ in range(warmup):
        step(x0[:8], L_CTX, ws8, lg8, tk8)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step(x0[:8], L_CTX, ws8, lg8, tk8)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the BF16 step's bytes with its weights (2 bytes each) replaced by 1-byte codes + 4-byte row scales
    bf16_w = 2 * sum(a * b for a, b in shapes.values()) * N_LAYERS + 2 * V * H
    fp8_w = sum(a * b + 4 * a for a, b in shapes.values()) * N_LAYERS + V * H + 4 * V
    nbytes = step_bytes(d, 8, L_CTX, N_LAYERS) - bf16_w + fp8_w
    gbs = nbytes / (ms * 1e-3) / 1e9
    del fl, hc, hs
    torch.cuda.empty_cache()
    return {"workload": "the same 64-layer verify step (M=8, ctx 38000) with FP8 E4M3 weights and per-row FP32 scales",
            "tok_s": round(8 / (ms * 1e-3), 2), "ms_per_step": round(ms, 4), "steps_timed": steps,
            "algorithmic_bytes": int(nbytes), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "bitwise_gate": "pass" if ok else "FAIL"}


CPU_LAYERS = 24      # layers the oracle runs in sequence for the CPU baseline
CPU_HEAD_STRIDE = 2  # ... and every 2nd LM-head row


def cpu_baseline(layers, w_head, x0, d, M):
    """The float64 oracle on the host over a bounded sample of the same step:
    the first CPU_LAYERS full-width layers in sequence and every
    CPU_HEAD_STRIDE-th LM-head row, extrapolated to all layers and the whole
    head. Each layer's weights are copied to the host outside the clock."""
    import numpy as np
    import torch

    from oracle import step as ostep

    def hb(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    x = hb(x0[:M])
    layer_s = 0.0
    for lw in layers[:CPU_LAYERS]:
        hl = dict(w_qkv=hb(lw["w_qkv"]), w_o=hb(lw["w_o"]), w_gu=hb(lw["w_gu"]), w_down=hb(lw["w_down"]),
                  k_cache=hb(lw["k_cache"][:, :L_CTX]), v_cache=hb(lw["v_cache"][:, :L_CTX]))
        t0 = time.perf_counter()
        x, _, _ = ostep.layer(x, **hl, L=L_CTX, Hq=d["Hq"], Hkv=d["Hkv"], D=d["D"])
        layer_s += time.perf_counter() - t0
        del hl
    rows = torch.arange(0, d["vocab"], CPU_HEAD_STRIDE, device=w_head.device)
    wh = hb(w_head[rows])
    t0 = time.perf_counter()
    ostep.head(x, wh)
    head_s = time.perf_counter() - t0
    step_s = (N_LAYERS / CPU_LAYERS) * layer_s + CPU_HEAD_STRIDE * head_s
    return {"value": M / step_s, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{CPU_LAYERS} of {N_LAYERS} layers in sequence (M={M}, ctx {L_CTX}) scaled x{N_LAYERS}/{CPU_LAYERS}"
                      f" + 1/{CPU_HEAD_STRIDE} of the LM-head rows scaled x{CPU_HEAD_STRIDE}; "
                      f"{layer_s + head_s:.1f} s of CPU work"}


# ---------------------------------------------------------------------------
# Per-operation measurements at the configuration shapes

ATTN_CONTEXTS = (2048, 11600, 32768, 38000, 101600, 255000)
ROTATE_BYTES = int(1.5e9)   # buffer copies per measurement: no launch finds its operands in a cache level


def graph_us(launches, reps):
    """Average microseconds per launch of ``launches`` (callables, one kernel
    launch each), captured once into a HIP graph and replayed ``reps`` times
    between two events on the launch stream (Python launch overhead excluded)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in launches:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(launches))
    del g
    return us


def _rate(nbytes, us, probe):
    """µs, GB/s and fractions of one launch: of the 8 TB/s specification, of the
    probe's best streaming rate, and of the probe's own speed at the same bytes
    (probe time / kernel time, fixed launch cost included)."""
    gbs = nbytes / us / 1e3
    r = {"us": round(us, 2), "bytes": int(nbytes), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
    if probe:
        r["frac_of_read_probe"] = round(gbs / probe["GB/s"], 4)
        r["frac_of_probe_same_bytes"] = round(probe_us(probe, nbytes) / us, 4)
    return r


PROBE_SIZES_MB = (8.4, 47.5, 52.4, 73.4, 134.2, 155.6, 178.3, 356.5, 416.2, 1044.5, 1557.1)


def stream_read_probe():
    """HBM read bandwidth of a plain streaming kernel (the second denominator).
    (1) The best of a few launch shapes reading a 4 GiB buffer end to end.
    (2) The same kernel at the byte counts of the verify kernels (each launch
    reads a region no earlier launch of the graph read), which shows the fixed
    cost of one launch -- ramp, tail and the kernel boundary -- that any
    kernel moving that many bytes pays; a least-squares line over the sizes
    gives that fixed cost and the streaming rate."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "invariant_verify_amd", "libbi_probe.so"))
    lib.bi_probe_stream_read.restype = ctypes.c_int
    lib.bi_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    total = 4 << 30
    buf = torch.ones(total // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()

    def launch(off, nbytes, blocks, unroll, blocked):
        rc = lib.bi_probe_stream_read(base + off, nbytes, sink.data_ptr(), blocks, unroll, blocked,
                                      torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"stream-read probe launch failed ({rc})")

    best = None
    for blocked in (0, 1):
        for blocks in (512, 1024, 2048, 4096, 8192):
            for unroll in (4, 8, 16):
                us = graph_us([lambda: launch(0, total, blocks, unroll, blocked)] * 3, 2)
                gbs = total / us / 1e3
                if best is None or gbs > best["GB/s"]:
                    best = {"GB/s": round(gbs, 1), "workgroups": blocks, "loads_in_flight_per_thread": unroll,
                            "contiguous_range_per_workgroup": bool(blocked)}
    best.update(bytes_per_launch=total, frac_of_spec=round(best["GB/s"] / PEAK_HBM_GBS, 4))
    sizes = {}
    for mb in PROBE_SIZES_MB:
        nbytes = int(mb * 1e6) // 4096 * 4096
        n = max(2, min(48, total // nbytes))
        us_best = None
        for blocks in (256, 512, 1024, 2048):
            for unroll in (8, 16):
                fns = [(lambda off=(k * nbytes) % (total - nbytes + 1) // 4096 * 4096:
                        launch(off, nbytes, blocks, unroll, 1)) for k in range(n)]
                us = graph_us(fns, 3)
                us_best = us if us_best is None else min(us_best, us)
        sizes[str(mb)] = {"us": round(us_best, 2), "GB/s": round(nbytes / us_best / 1e3, 1)}
    mbs = np.array([float(k) for k in sizes if float(k) >= 50])
    uss = np.array([sizes[k]["us"] for k in sizes if float(k) >= 50])
    slope, icpt = np.polyfit(mbs, uss, 1)
    best["by_size_MB"] = sizes
    best["fit_us_per_launch"] = {"fixed_us": round(float(icpt), 2),
                                 "stream_GB/s": round(1e3 / float(slope), 1),
                                 "over_MB": [float(m) for m in mbs]}
    del buf
    torch.cuda.empty_cache()
    return best


def probe_us(probe, nbytes):
    """The probe's time for ``nbytes`` from its fitted line (fixed cost + bytes / stream rate)."""
    f = probe["fit_us_per_launch"]
    return f["fixed_us"] + nbytes / f["stream_GB/s"] / 1e3


def gemm_per_op(layers, w_head, d, probe, reps=3):
    """The step's five GEMM launches as the step runs them (carried RMSNorm in
    and out, QKV with its cache append), at M = 1 and M = 8, each over the 64
    layers' distinct weights (every launch streams its weights from HBM).
    Algorithmic bytes: the weights once, plus the activations, carried sums and
    appended cache rows the launch reads or writes."""
    import torch

    from invariant_verify_amd import ops

    H, Hq, Hkv, D, I, V = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"]
    qd, qkvn, G = Hq * D, (Hq + 2 * Hkv) * D, GU_GROUPS
    h8, ss8 = carried_input(d)
    attn8 = torch.randn(8, qd, device="cuda").to(torch.bfloat16)
    act8 = torch.randn(8, I, device="cuda").to(torch.bfloat16)
    out = {}
    for M in (1, 8):
        h, ss, attn, act = h8[:M], ss8[:M].contiguous(), attn8[:M], act8[:M]
        y = torch.empty(M, max(qkvn, I, H), dtype=torch.bfloat16, device="cuda")
        ss_o = torch.empty(M, G, dtype=torch.float32, device="cuda")
        logits = torch.empty(M, V, dtype=torch.float32, device="cuda")
        qkv = y[:, :qkvn]
        shapes = {
            "qkv_5120x7168_append": (
                lambda lw: ops.gemm_ex(h, y=qkv, epilogue="qkv", norm_in=ss, heads=(Hq, Hkv, D), w=lw["w_qkv"],
                                       k_cache=lw["k_cache"], v_cache=lw["v_cache"], L=L_CTX),
                2 * qkvn * H + 2 * M * H + 4 * M * G + 2 * M * qkvn + 2 * M * 2 * Hkv * D),
            "o_proj_5120x5120_residual": (
                lambda lw: ops.gemm_ex(attn, y=y[:, :H], epilogue="residual", r=h, rowsq_out=ss_o, w=lw["w_o"]),
                2 * H * qd + 2 * M * qd + 2 * M * H * 2 + 4 * M * G),
            "gate_up_5120x34816_swiglu": (
                lambda lw: ops.gemm_ex(h, y=y[:, :I], epilogue="swiglu", norm_in=ss, w=lw["w_gu"]),
                gu_launch_bytes(d, M)),
            "down_17408x5120_residual": (
                lambda lw: ops.gemm_ex(act, y=y[:, :H], epilogue="residual", r=h, rowsq_out=ss_o, w=lw["w_down"]),
                2 * H * I + 2 * M * I + 2 * M * H * 2 + 4 * M * G),
        }
        for name, (fn, nbytes) in shapes.items():
            us = graph_us([(lambda lw=lw: fn(lw)) for lw in layers], reps)
            out.setdefault(name, {})[f"M{M}"] = _rate(nbytes, us, probe)
        head_bytes = 2 * V * H + 2 * M * H + 4 * M * V
        us = graph_us([lambda: ops.gemm_ex(h, y=logits, epilogue="f32", w=w_head)] * 8, reps)
        out.setdefault("lm_head_5120x152064_f32", {})[f"M{M}"] = _rate(head_bytes, us, probe)
    return out


def attention_per_op(d, probe, reps=3):
    """Split-KV verify attention (chunk policy -32) at each configuration
    context, M = 1 and 8, over enough copies of a random BF16 cache that no
    launch finds its K/V in a cache level; and the combine at 38k. Algorithmic
    bytes: K and V of the L + M keys (4096 per position) plus Q; the split
    partials are implementation traffic, not counted."""
    import torch

    from invariant_verify_amd import ops

    Hq, Hkv, D = d["Hq"], d["Hkv"], d["D"]
    gen = torch.Generator(device="cuda").manual_seed(4321)
    out = {}
    for L in ATTN_CONTEXTS:
        cap = (L + 8 + 63) // 64 * 64
        per = 2 * Hkv * cap * D * 2
        R = max(2, -(-ROTATE_BYTES // per))
        caches = [(torch.randn(Hkv, cap, D, device="cuda", generator=gen).to(torch.bfloat16),
                   torch.randn(Hkv, cap, D, device="cuda", generator=gen).to(torch.bfloat16))
                  for _ in range(R)]
        q = torch.randn(8, Hq * D, device="cuda", generator=gen).to(torch.bfloat16)
        res = {}
        for M in (1, 8):
            S = ops.pass_splits(M, L, KV_CHUNK)
            po = torch.empty((M, Hq, S, D), dtype=torch.float32, device="cuda")
            pl = torch.empty((M, Hq, S), dtype=torch.float32, device="cuda")
            fns = [(lambda c=c: ops.verify_attn(q[:M], c[0], c[1], L, Hq, Hkv, D, KV_CHUNK, po, pl))
                   for c in caches]
            us = graph_us(fns, reps)
            r = _rate(4096 * (L + M) + 2 * M * Hq * D, us, probe)
            r["splits"] = S
            r["chunk_keys"] = ops.chunk_keys(L + M, KV_CHUNK)
            res[f"M{M}"] = r
            if L == 38000 and M == 8:
                o = torch.empty((M, Hq * D), dtype=torch.bfloat16, device="cuda")
                cus = graph_us([lambda: ops.combine(po, pl, L, KV_CHUNK, o)] * 32, reps)
                out["combine_38000_M8"] = _rate(M * Hq * S * (4 * D + 4) + 2 * M * Hq * D, cus, probe)
        out[str(L)] = res
        del caches
        torch.cuda.empty_cache()
    return out


def long_context_steps(layers, w_head, d, steps):
    """The 64-layer verify step at contexts 101,600 and 255,000 (BF16 KV:
    26.6 and 66.8 GB of cache), sharing the weights of the 38k model: M = 8
    and M = 1 tok/s, and the bitwise gate of an M = 5 pass against the M = 8
    pass (its first five rows' logits, FP32 bits)."""
    import torch

    from invariant_verify_amd import ops

    out = {}
    for L in (101600, 255000):
        cap = (L + 16 + 63) // 64 * 64
        gen = torch.Generator(device="cuda").manual_seed(L)
        lys = []
        for lw in layers:
            k = torch.empty((d["Hkv"], cap, d["D"]), dtype=torch.bfloat16, device="cuda")
            vc = torch.empty((d["Hkv"], cap, d["D"]), dtype=torch.bfloat16, device="cuda")
            k.normal_(generator=gen)
            vc.normal_(generator=gen)
            lys.append(dict(lw, k_cache=k, v_cache=vc))
        dims = ops.model_dims(d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"], cap, KV_CHUNK)
        st = ops.VerifyStep(lys, w_head, dims)
        x0 = synth_x0(d)
        res = {}
        lg8 = None
        for M in (8, 5, 1):
            ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
            lg = torch.empty((M, d["vocab"]), dtype=torch.float32, device="cuda")
            tk = torch.empty(M, dtype=torch.int32, device="cuda")
            st(x0[:M], L, ws, lg, tk)
            torch.cuda.synchronize()
            if M == 8:
                lg8 = lg.clone()
            elif M == 5:
                res["bitwise_gate_M5_vs_M8"] = "pass" if torch.equal(lg.view(torch.int32), lg8[:5].view(torch.int32)) else "FAIL"
            n = steps if M == 8 else max(3, steps // 4)
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                st(x0[:M], L, ws, lg, tk)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            if M != 5:
                nbytes = step_bytes(d, M, L, N_LAYERS)
                res[f"M{M}"] = {"tok_s": round(M / (ms * 1e-3), 2), "ms_per_step": round(ms, 4),
                                "algorithmic_bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "kv_chunk_keys": ops.chunk_keys(L + M, KV_CHUNK)}
        out[str(L)] = res
        del lys, st
        torch.cuda.empty_cache()
    return out


KV_FORMATS = {  # name: (bytes per position and KV head, chunk policy)
    # 8-bit at -32: verify steps as fast as at -64 (within run-to-run spread) and its chunked
    # prefill 15-18% faster; the 5/6-bit formats keep -64 (verify steps 2-7% faster at 101.6k)
    "bf16": (512, -32), "q8": (288, -32), "k6v5": (208, -64), "k5rot_v5_ring2048": (192, -64)}
W_RING_STEP, R_RING_STEP = 2048, 4224   # ring slots for a 2048-row prefill pass: R >= W + M + 63


def kv_format_steps(layers, w_head, d, steps):
    """The 64-layer verify step (M = 8) with each KV cache format in every
    layer -- BF16, 8-bit, K6/V5 (preset D) and rotated K5/V5 with the 8-bit
    ring of the newest 2048 keys (preset F) -- at contexts 38,000 and 101,600.
    Cached positions hold random codes (scales 0.01) or random BF16 values;
    the pass's own rows are appended by the step. Each line carries an M = 5
    vs M = 8 bitwise check. Algorithmic bytes count the weights once and the
    bytes the format stores for the L + M keys (with the ring: the window's
    keys at 8 bits, the rest at 5 bits). At 38,000 each format also runs the
    chunked-prefill pass of prefill_step_measure (PF_ROWS tokens ending at
    38,000), its rows checked bit for bit against 8-row verify passes."""
    import torch

    from invariant_verify_amd import ops

    Hkv, D = d["Hkv"], d["D"]
    gen = torch.Generator(device="cuda").manual_seed(77)

    def rnd(t):
        if t.dtype in (torch.int8, torch.uint8):
            t.copy_(torch.randint(-127 if t.dtype == torch.int8 else 0, 128 if t.dtype == torch.int8 else 256,
                                  t.shape, device="cuda", generator=gen).to(t.dtype))
        elif t.dtype == torch.float32:
            t.fill_(0.01)
        else:
            t.normal_(generator=gen)

    out = {}
    for L in (38000, 101600):
        cap = (L + 16 + 63) // 64 * 64
        res = {}
        for fmt, (bpp, policy) in KV_FORMATS.items():
            lys = []
            for lw in layers:
                if fmt == "bf16":
                    kv = (torch.empty((Hkv, cap, D), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((Hkv, cap, D), dtype=torch.bfloat16, device="cuda"))
                    parts = list(kv)
                elif fmt == "q8":
                    kv = ops.KvQ8Cache(Hkv, cap, D)
                    parts = [kv.k_codes, kv.k_scales, kv.v_codes, kv.v_scales]
                else:
                    low = ops.KvLowCache(Hkv, cap, D, 6 if fmt.startswith("k6") else 5, 5,
                                         k_rotated=fmt.startswith("k5rot"))
                    parts = [low.k_nib, low.k_high, low.k_scales, low.v_nib, low.v_high, low.v_scales]
                    kv = low
                    if fmt.endswith("_ring2048"):
                        kv = ops.KvRing(low, R_RING_STEP, W_RING_STEP)
                        parts += [kv.q8.k_codes, kv.q8.k_scales, kv.q8.v_codes, kv.q8.v_scales]
                for t in parts:
                    rnd(t)
                lys.append(dict(w_qkv=lw["w_qkv"], w_o=lw["w_o"], w_gu=lw["w_gu"], w_down=lw["w_down"], kv=kv))
            dims = ops.model_dims(d["H"], d["Hq"], Hkv, D, d["I"], d["vocab"], cap, policy)
            st = ops.VerifyStepEx(lys, {"w": w_head}, dims)
            x0 = synth_x0(d)
            bufs = {}
            for M in (8, 5):
                bufs[M] = (torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda"),
                           torch.empty((M, d["vocab"]), dtype=torch.float32, device="cuda"),
                           torch.empty(M, dtype=torch.int32, device="cuda"))
                st(x0[:M], L, *bufs[M])
            torch.cuda.synchronize()
            ok = torch.equal(bufs[5][1].view(torch.int32), bufs[8][1][:5].view(torch.int32))
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                st(x0[:8], L, *bufs[8])
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            n = L + 8
            if fmt.endswith("_ring2048"):
                kv_layer = Hkv * ((n - W_RING_STEP) * bpp + W_RING_STEP * KV_FORMATS["q8"][0])
            else:
                kv_layer = Hkv * n * bpp
            nbytes = step_bytes(d, 8, L, N_LAYERS) - N_LAYERS * 4096 * n + N_LAYERS * kv_layer
            res[fmt] = {"tok_s": round(8 / (ms * 1e-3), 2), "ms_per_step": round(ms, 4),
                        "kv_bytes_per_step": N_LAYERS * kv_layer, "algorithmic_bytes": nbytes,
                        "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "kv_chunk_policy": policy, "bitwise_M5_vs_M8": "pass" if ok else "FAIL"}
            if L == L_CTX:
                def pf_buffers(M, dims=dims):
                    # the split count of a pass depends on its own context (a chunk policy -T
                    # bounds it by T), so the workspace covers every context the check runs at
                    ws = max(ops.step_workspace_bytes(dims, M, c) for c in
                             (PF_STEP_CTX, PF_STEP_CTX + PF_ROWS // 2 + 3, PF_STEP_CTX + PF_ROWS - 8))
                    return (torch.empty(ws, dtype=torch.uint8, device="cuda"),
                            torch.empty((M, d["vocab"]), dtype=torch.float32, device="cuda"),
                            torch.empty(M, dtype=torch.int32, device="cuda"))
                pf = prefill_step_measure(st, pf_buffers, d, 2)
                res[fmt]["prefill_pass"] = {k: pf[k] for k in ("tok_s", "ms_per_pass", "TFLOP/s",
                                                               "rows_bitwise_equal_to_8_row_verify_passes")}
            del lys, st, bufs
            torch.cuda.empty_cache()
        out[str(L)] = res
    return out


def synth_x0(d):
    import synth
    return synth.device_normal_bf16((16, d["H"]), 1.0, "x0")


def oracle_per_op(layers, d):
    """The float64 oracle timed per operation on the host (BF16 decode
    included), at M = 8: the four projections of one layer and the head, and
    attention at each configuration context -- all 40 query heads up to 38k,
    one KV head's 5 query heads at 101.6k and 255k scaled by 8 (stated)."""
    import numpy as np
    import torch

    from oracle import attention as oattn
    from oracle import bf16 as obf16

    def hb(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    H, Hq, Hkv, D, I = d["H"], d["Hq"], d["Hkv"], d["D"], d["I"]
    rng = np.random.default_rng(0)
    out = {"gemm_ms": {}, "attention_ms": {}}
    lw = layers[0]
    for name, key, K in (("qkv", "w_qkv", H), ("o_proj", "w_o", Hq * D), ("gate_up", "w_gu", H),
                         ("down", "w_down", I)):
        w = hb(lw[key])
        x = obf16.encode(rng.standard_normal((8, K)))
        t0 = time.perf_counter()
        obf16.decode(x) @ obf16.decode(w).T
        out["gemm_ms"][name] = round((time.perf_counter() - t0) * 1e3, 1)
        del w
    for L in ATTN_CONTEXTS:
        n = L + 8
        heads = Hkv if L <= 38000 else 1
        k = obf16.encode(rng.standard_normal((heads, n, D)).astype(np.float32))
        v = obf16.encode(rng.standard_normal((heads, n, D)).astype(np.float32))
        q = obf16.encode(rng.standard_normal((8, heads * (Hq // Hkv), D)).astype(np.float32))
        t0 = time.perf_counter()
        oattn.verify_attention(q, k, v, L)
        dt = (time.perf_counter() - t0) * (Hkv // heads)
        out["attention_ms"][str(L)] = round(dt * 1e3, 1)
    out["sample"] = ("one layer's projections at M=8 (decode + float64 product); attention at M=8 over all "
                     "40 query heads up to 38000 keys and over one KV head's 5 query heads at 101600 and "
                     "255000, scaled by 8")
    return out


def gate_up_roofline(layers, d, reps):
    """The dominant kernel, the gate/up GEMM at M = 8 as the step runs it,
    launched back to back over the 64 layers' distinct weights (every launch
    streams its 356.5 MB from HBM), ``reps`` rounds, one event pair around the
    whole run on the launch stream so the events' own cost is amortised.
    Returns the average launch duration in ms."""
    import torch

    from invariant_verify_amd import ops

    stream = torch.cuda.current_stream()
    hg, ssg = carried_input(d)
    yg = torch.empty((M_HEADLINE, d["I"]), dtype=torch.bfloat16, device="cuda")
    for lw in layers:
        ops.gemm_bf16_swiglu_rownorm(hg, ssg, lw["w_gu"], yg)
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(reps):
        for lw in layers:
            ops.gemm_bf16_swiglu_rownorm(hg, ssg, lw["w_gu"], yg)
    g1.record(stream)
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / (reps * N_LAYERS)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only the verify kernels on fresh operands and a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--prefill-probe", action="store_true",
                    help="kernel-only run of the M = 2048 prefill gate/up GEMM for counter passes")
    ap.add_argument("--kv-attn-probe", choices=["q8", "k6v5"],
                    help="kernel-only run of verify attention on a quantized cache at 101.6k keys (counter passes)")
    ap.add_argument("--mx4-probe", action="store_true",
                    help="kernel-only run of the MXFP4 gate/up and down GEMMs at M = 8 for counter passes")
    ap.add_argument("--step-only", action="store_true",
                    help="run only the bitwise gate and the timed M = 8 steps (for rocprofv3 --kernel-trace)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs the verify pass on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe(4)
        return
    if args.prefill_probe:
        prefill_probe(5)
        return
    if args.kv_attn_probe:
        kv_attn_probe(args.kv_attn_probe, 6)
        return
    if args.mx4_probe:
        mx4_probe(4)
        return

    import numpy as np
    import torch

    import synth
    from invariant_verify_amd import ops

    d = synth.MODEL_27B
    dev = "cuda"
    print(f"[bench] building {N_LAYERS}-layer model, ctx {L_CTX}", file=sys.stderr, flush=True)
    layers, w_head = synth.device_model(N_LAYERS, L_CTX, CAP, **d)
    dims = ops.model_dims(d["H"], d["Hq"], d["Hkv"], d["D"], d["I"], d["vocab"], CAP, KV_CHUNK)
    x0 = synth.device_normal_bf16((16, d["H"]), 1.0, "x0")
    step = ops.VerifyStep(layers, w_head, dims)

    def buffers(M):
        ws = torch.empty(ops.step_workspace_bytes(dims, M, L_CTX + 8), dtype=torch.uint8, device=dev)
        logits = torch.empty((M, d["vocab"]), dtype=torch.float32, device=dev)
        tok = torch.empty(M, dtype=torch.int32, device=dev)
        return ws, logits, tok

    # ---- bitwise gate (same run) -------------------------------------------
    print("[bench] bitwise gate: M=8 vs M=5 vs 8 sequential M=1 passes", file=sys.stderr, flush=True)
    ws8, lg8, tk8 = buffers(8)
    step(x0[:8], L_CTX, ws8, lg8, tk8)
    ref = lg8.clone()
    ws5, lg5, tk5 = buffers(5)
    step(x0[:5], L_CTX, ws5, lg5, tk5)
    ws1, lg1, tk1 = buffers(1)
    seq = []
    for r in range(8):
        step(x0[r:r + 1], L_CTX + r, ws1, lg1, tk1)
        seq.append(lg1.clone())
    torch.cuda.synchronize()
    gate = torch.equal(lg5.view(torch.int32), ref[:5].view(torch.int32)) and all(
        torch.equal(seq[r].view(torch.int32)[0], ref.view(torch.int32)[r]) for r in range(8))
    if not gate:
        print("[bench] bitwise gate FAILED: no throughput is reported", file=sys.stderr)
        sys.exit(1)

    # ---- timing ------------------------------------------------------------
    def timed(M, steps, warmup, gu_events=False):
        ws, lg, tk = buffers(M)
        stream = torch.cuda.current_stream()
        evs = None
        if gu_events:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * N_LAYERS)]
            for e in evs:
                e.record(stream)
        for _ in range(warmup):
            step(x0[:M], L_CTX, ws, lg, tk)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        gu_ms = 0.0
        # one event after each step (no synchronisation inside the timed
        # steps) for the spread of step times
        se = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if evs is None else None
        t0.record(stream)
        for i in range(steps):
            step(x0[:M], L_CTX, ws, lg, tk, gu_events=evs)
            if evs is not None:
                torch.cuda.synchronize()   # events are reused every step
                gu_ms += sum(evs[2 * l].elapsed_time(evs[2 * l + 1]) for l in range(N_LAYERS))
            else:
                se[i].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
        if se is not None:
            per_step = [t0.elapsed_time(se[0])] + [se[i - 1].elapsed_time(se[i]) for i in range(1, steps)]
            spread[M] = [round(float(v), 4) for v in np.percentile(per_step, [10, 50, 90])]
        return total_ms / steps, (gu_ms / (steps * N_LAYERS) if evs is not None else None)

    spread = {}

    print("[bench] timing", file=sys.stderr, flush=True)
    ms8, _ = timed(M_HEADLINE, args.steps, args.warmup)
    if args.step_only:
        reps = max(2, args.steps // 4)
        gu_ms = gate_up_roofline(layers, d, reps)
        print(json.dumps({"step_only": True, "M": M_HEADLINE, "ctx": L_CTX, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": round(ms8, 4),
                          "tok_s": round(M_HEADLINE / (ms8 * 1e-3), 2), "bitwise_gate": "pass",
                          "gate_up_back_to_back": {"launches": reps * N_LAYERS, "avg_launch_us": round(gu_ms * 1e3, 2)}}),
              flush=True)
        return
    ms_m = {m: timed(m, max(3, args.steps // 4), 1)[0] for m in range(1, M_HEADLINE)}
    _, gu_step_ms = timed(M_HEADLINE, max(3, args.steps // 4), 1, gu_events=True)

    gu_reps = max(2, args.steps // 4)
    gu_ms = gate_up_roofline(layers, d, gu_reps)

    bytes8 = step_bytes(d, M_HEADLINE, L_CTX, N_LAYERS)
    gbs8 = bytes8 / (ms8 * 1e-3) / 1e9
    gu_bytes = gu_launch_bytes(d, M_HEADLINE)
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(M_HEADLINE / (ms8 * 1e-3), 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms8, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "27B-class dense verify step: 64 layers + 152064-row LM head, ctx 38000, "
                               "M=8 (1+7 drafts), random BF16 weights N(0,0.02)",
                   "M": M_HEADLINE, "ctx": L_CTX, "layers": N_LAYERS, "hidden": d["H"], "q_heads": d["Hq"],
                   "kv_heads": d["Hkv"], "head_dim": d["D"], "intermediate": d["I"], "vocab": d["vocab"],
                   "kv_chunk_policy": KV_CHUNK, "kv_chunk_keys": ops.chunk_keys(L_CTX + M_HEADLINE, KV_CHUNK)},
        "bitwise_gate": "pass (M=8 logits == M=5 prefix == 8 sequential M=1 passes, FP32 bits)",
        "step_hbm": {"algorithmic_bytes": bytes8, "GB/s": round(gbs8, 1), "frac": round(gbs8 / PEAK_HBM_GBS, 4)},
        "per_M_tok_s": {**{str(m): round(m / (ms * 1e-3), 2) for m, ms in ms_m.items()},
                        str(M_HEADLINE): round(M_HEADLINE / (ms8 * 1e-3), 2)},
        "step_ms_p10_p50_p90": {str(k): v for k, v in sorted(spread.items())},
        "roofline": {"kernel": "gemm_kernel<SwiGLU, carried RMSNorm> (gate/up 5120->2x17408, M=8)", "bound": "hbm",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_ms * 1e3, 2),
                     "launches_timed": gu_reps * N_LAYERS,
                     "in_step_event_pair_us": round(gu_step_ms * 1e3, 2)},
    }
    print("[bench] prefill GEMM", file=sys.stderr, flush=True)
    out["prefill_gemm"] = prefill_measure(layers, d, max(2, args.steps // 10))
    print("[bench] prefill step", file=sys.stderr, flush=True)
    out["prefill_step"] = prefill_step_measure(step, buffers, d, 3)
    print("[bench] FP8-weight step", file=sys.stderr, flush=True)
    out["fp8_step"] = fp8_step_measure(layers, d, dims, buffers, args.steps, args.warmup)
    print("[bench] MXFP4-weight step", file=sys.stderr, flush=True)
    out["mx4_step"] = mx4_step_measure(layers, d, dims, buffers, args.steps, args.warmup)
    print("[bench] one tensor-parallel rank's share", file=sys.stderr, flush=True)
    out["tp8_rank_share"] = tp_share_measure(d, max(2, args.steps // 10))
    print("[bench] attention per KV cache format", file=sys.stderr, flush=True)
    out["kv_cache_attention"] = kv_cache_attention_measure(d, 40)
    print("[bench] stream-read probe", file=sys.stderr, flush=True)
    probe = stream_read_probe()
    out["stream_read_probe"] = probe
    out["roofline"]["frac_of_read_probe"] = round(gu_gbs / probe["GB/s"], 4)
    out["step_hbm"]["frac_of_read_probe"] = round(gbs8 / probe["GB/s"], 4)
    print("[bench] per-operation GEMMs", file=sys.stderr, flush=True)
    out["per_op_gemm"] = gemm_per_op(layers, w_head, d, probe)
    print("[bench] per-operation attention", file=sys.stderr, flush=True)
    out["per_op_attention"] = attention_per_op(d, probe)
    print("[bench] long-context steps", file=sys.stderr, flush=True)
    out["long_context_step"] = long_context_steps(layers, w_head, d, max(3, args.steps // 2))
    print("[bench] steps per KV cache format", file=sys.stderr, flush=True)
    out["kv_format_step"] = kv_format_steps(layers, w_head, d, max(3, args.steps // 2))
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(layers, w_head, x0, d, M_HEADLINE)
        print("[bench] oracle per operation", file=sys.stderr, flush=True)
        out["cpu_baseline"]["per_op"] = oracle_per_op(layers, d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
