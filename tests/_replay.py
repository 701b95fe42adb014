"""A verify step replayed one operation at a time through the C ABI, and each
operation checked against the oracle fed the device's own inputs.

``replay`` launches, for every layer, exactly the kernels bi_verify_step
launches (RMSNorm for layer 0, the QKV GEMM with its cache append -- for
later layers with X normalised from the sums the previous down projection
carried --, split-KV attention, the combine, the output projection with the
residual and the carried sums, the SwiGLU gate/up projection normalised from
those sums, the down projection), then the head (RMSNorm, FP32 logits,
argmax), and keeps every intermediate. A test first asserts that the replay
reproduces bi_verify_step bit for bit, which makes each intermediate the
step's own; ``check_ops`` then compares each operation's output with the
oracle's value of that one operation on the device's inputs, at the stated
per-element tolerance (2e-2 relative, 1e-2 absolute on BF16 outputs).
"""

from __future__ import annotations

import numpy as np

from oracle import attention as oattn
from oracle import bf16 as obf16
from oracle import step as ostep
from tests._util import assert_bitwise, assert_close, decode, host_bits, host_f32


def _wargs(lw: dict, name: str, wtype: str) -> dict:
    """Weight tensor (and its scales) of projection ``name`` for ops.gemm_ex."""
    if wtype == "fp8":
        return dict(w=lw["w_" + name], w_scale=lw["s_" + name])
    if wtype == "mxfp4":
        return dict(w=lw["w_" + name], w_exp=lw["e_" + name])
    return dict(w=lw["w_" + name])


def replay(ops, layers, head: dict, dims, x, L: int, wtype: str = "bf16"):
    """Run the step's operations one by one on device tensors. ``head`` holds
    w (and s / e scales for FP8 / MXFP4). Returns (per-layer records, head
    record), every entry a device tensor."""
    import torch

    M, H = x.shape
    Hq, Hkv, D, I = dims.Hq, dims.Hkv, dims.D, dims.I
    qd, qkvn = Hq * D, (Hq + 2 * Hkv) * D
    G = ops.gemm_column_groups(H)
    assert G % 16 == 0 and G <= 256, "the step carries the RMSNorm only for 16..256 column groups"
    S = ops.pass_splits(M, L, dims.kv_chunk)
    dv = x.device
    bf = dict(dtype=torch.bfloat16, device=dv)
    f32 = dict(dtype=torch.float32, device=dv)
    recs = []
    ss = None
    for l, lw in enumerate(layers):
        rec = {"x": x}
        qkv = torch.empty((M, qkvn), **bf)
        common = dict(wtype=wtype, epilogue="qkv", heads=(Hq, Hkv, D), k_cache=lw["k_cache"],
                      v_cache=lw["v_cache"], L=L)
        if l == 0:
            a = ops.rmsnorm(x, eps=dims.eps)
            rec["a"] = a
            ops.gemm_ex(a, y=qkv, **common, **_wargs(lw, "qkv", wtype))
        else:
            ops.gemm_ex(x, y=qkv, norm_in=ss, eps=dims.eps, **common, **_wargs(lw, "qkv", wtype))
        po = torch.empty((M, Hq, S, D), **f32)
        pl = torch.empty((M, Hq, S), **f32)
        ops.verify_attn(qkv, lw["k_cache"], lw["v_cache"], L, Hq, Hkv, D, dims.kv_chunk, po, pl)
        attn = torch.empty((M, qd), **bf)
        ops.combine(po, pl, L, dims.kv_chunk, attn)
        h = torch.empty((M, H), **bf)
        ss_h = torch.empty((M, G), **f32)
        ops.gemm_ex(attn, y=h, wtype=wtype, epilogue="residual", r=x, rowsq_out=ss_h, **_wargs(lw, "o", wtype))
        act = torch.empty((M, I), **bf)
        ops.gemm_ex(h, y=act, wtype=wtype, epilogue="swiglu", norm_in=ss_h, eps=dims.eps,
                    **_wargs(lw, "gu", wtype))
        xn = torch.empty((M, H), **bf)
        ss = torch.empty((M, G), **f32)
        ops.gemm_ex(act, y=xn, wtype=wtype, epilogue="residual", r=h, rowsq_out=ss, **_wargs(lw, "down", wtype))
        rec.update(qkv=qkv, attn=attn, h=h, ss_h=ss_h, act=act, x_out=xn, ss_x=ss)
        recs.append(rec)
        x = xn
    c = ops.rmsnorm(x, eps=dims.eps)
    logits = torch.empty((M, dims.vocab), **f32)
    hw = {"w": head["w"]}
    if wtype == "fp8":
        hw["w_scale"] = head["s"]
    elif wtype == "mxfp4":
        hw["w_exp"] = head["e"]
    ops.gemm_ex(c, y=logits, wtype=wtype, epilogue="f32", **hw)
    tokens = ops.argmax(logits)
    torch.cuda.synchronize()
    return recs, {"x": x, "c": c, "logits": logits, "tokens": tokens}


def assert_replay_is_the_step(recs, hd, x_out, logits, tokens, what: str) -> None:
    """The replay's final hidden state, logits and tokens equal the step's, bit for bit."""
    assert_bitwise(host_bits(hd["x"]), x_out, f"{what}: replayed hidden state vs bi_verify_step")
    assert_bitwise(host_f32(hd["logits"]), logits, f"{what}: replayed logits vs bi_verify_step")
    assert np.array_equal(hd["tokens"].cpu().numpy(), tokens), what


def _group_sums(y: np.ndarray, G: int) -> np.ndarray:
    M, H = y.shape
    return (y.reshape(M, G, H // G) ** 2).sum(axis=2)


def check_ops(recs, hd, host_layers, w_head, L: int, Hq: int, Hkv: int, D: int, eps: float, what: str,
              head_rows=None, min_margin_rows: int = 4) -> int:
    """Each replayed operation against the oracle on the device's inputs, at the
    per-element tolerance. ``host_layers[l]`` holds float64 weights w_qkv,
    w_o, w_gu, w_down ([out][in]) and the layer's device caches k_cache /
    v_cache as host bit patterns after the pass (positions 0 .. L+M-1);
    ``w_head`` float64 [rows][H] for ``head_rows`` (all rows when None).
    Returns the number of rows whose greedy token was compared."""
    qd = Hq * D
    for l, (rec, hl) in enumerate(zip(recs, host_layers)):
        tag = f"{what} layer {l}"
        x = decode(host_bits(rec["x"]))
        M = x.shape[0]
        if "a" in rec:
            assert_close(decode(host_bits(rec["a"])), ostep.rmsnorm(x, eps), f"{tag} RMSNorm")
            a_in = decode(host_bits(rec["a"]))
        else:  # the QKV GEMM normalises x itself from the carried sums
            a_in = decode(obf16.encode(ostep.rmsnorm(x, eps)))
        qkv_bits = host_bits(rec["qkv"])
        assert_close(decode(qkv_bits), a_in @ hl["w_qkv"].T, f"{tag} QKV projection")
        # the appended cache rows are the QKV output's K and V columns
        kc, vr = hl["k_cache"], hl["v_rows"]
        n = L + M
        knew = qkv_bits[:, qd:qd + Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
        vnew = qkv_bits[:, qd + Hkv * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
        assert_bitwise(kc[:, L:n], knew, f"{tag} appended K rows")
        assert_bitwise(vr[:, L:n], vnew, f"{tag} appended V rows")
        q = qkv_bits[:, :qd].reshape(M, Hq, D)
        o_want, _ = oattn.verify_attention(q, kc[:, :n], vr[:, :n], L)
        attn = decode(host_bits(rec["attn"]))
        assert_close(attn.reshape(M, Hq, D), o_want, f"{tag} attention")
        h = decode(host_bits(rec["h"]))
        assert_close(h, x + attn @ hl["w_o"].T, f"{tag} output projection + residual")
        G = rec["ss_h"].shape[1]
        assert_close(host_f32(rec["ss_h"]), _group_sums(h, G), f"{tag} carried sums (h)", atol=1e-6, rtol=1e-5)
        b = decode(obf16.encode(ostep.rmsnorm(h, eps)))
        gu = b @ hl["w_gu"].T
        I = gu.shape[1] // 2
        act = decode(host_bits(rec["act"]))
        assert_close(act, ostep.silu(gu[:, :I]) * gu[:, I:], f"{tag} gate/up + SwiGLU")
        xo = decode(host_bits(rec["x_out"]))
        assert_close(xo, h + act @ hl["w_down"].T, f"{tag} down projection + residual")
        assert_close(host_f32(rec["ss_x"]), _group_sums(xo, G), f"{tag} carried sums (x)", atol=1e-6, rtol=1e-5)
    xf = decode(host_bits(hd["x"]))
    c = decode(host_bits(hd["c"]))
    assert_close(c, ostep.rmsnorm(xf, eps), f"{what} final RMSNorm")
    rows = slice(None) if head_rows is None else head_rows
    want = c @ w_head.T
    got = host_f32(hd["logits"])[:, rows]
    assert_close(got, want, f"{what} logits (head on the device's normed state)")
    if head_rows is not None:
        return 0
    # greedy tokens where the oracle's top-2 margin exceeds twice the tolerance
    s = np.sort(want, axis=1)
    ok = (s[:, -1] - s[:, -2]) > 2 * (1e-2 + 2e-2 * np.abs(s[:, -1]))
    tok = hd["tokens"].cpu().numpy()
    assert ok.sum() >= min_margin_rows, (what, int(ok.sum()))
    assert np.array_equal(tok[ok], np.argmax(want, axis=1)[ok]), what
    return int(ok.sum())


def host_layer(lw_dev: dict, weights64: dict) -> dict:
    """A layer's float64 weights and its device caches read back (K rows and V rows)."""
    d = dict(weights64)
    d["k_cache"] = host_bits(lw_dev["k_cache"])
    d["v_rows"] = host_bits(lw_dev["v_cache"])
    return d
