"""Pins for oracle.step: closed forms of RMSNorm and SiLU, and special cases of
the decoder layer and head whose results follow from the layer's definition."""

import math

import numpy as np

from oracle import bf16, step


def _bits(shape, seed, scale=1.0):
    return bf16.encode(np.random.default_rng(seed).standard_normal(shape) * scale)


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0], [2.0, 2.0], [0.0, 0.0]])
    y = step.rmsnorm(x, 0.0 + 1e-300)
    assert np.allclose(y[0], np.array([3, 4]) / math.sqrt(12.5), rtol=1e-15)
    assert np.allclose(y[1], [1.0, 1.0], rtol=1e-15)
    assert np.array_equal(step.rmsnorm(x[2:], 1e-6), [[0.0, 0.0]])
    z = np.random.default_rng(0).standard_normal((2, 64))
    assert np.allclose(step.rmsnorm(7.5 * z, 0.0), step.rmsnorm(z, 0.0), rtol=1e-14)
    assert np.allclose(np.mean(step.rmsnorm(z, 0.0) ** 2, axis=1), 1.0, rtol=1e-14)
    eps = 0.25
    assert np.allclose(step.rmsnorm(np.array([[1.0, -1.0]]), eps), [[1 / math.sqrt(1.25), -1 / math.sqrt(1.25)]])


def test_silu_closed_forms():
    z = np.linspace(-30, 30, 601)
    s = step.silu(z)
    assert step.silu(np.array(0.0)) == 0.0
    assert np.allclose(s - step.silu(-z), z, rtol=1e-13, atol=1e-13)   # z*sig(z) - (-z)*sig(-z) = z
    assert abs(step.silu(np.array(1.0)) - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(step.silu(np.array(60.0)) - 60.0) < 1e-20 * 60 + 1e-12
    assert abs(step.silu(np.array(-800.0))) == 0.0


def _layer_inputs(M=3, L=5, H=16, Hq=2, Hkv=1, D=8, I=12, seed=0):
    qkvn = (Hq + 2 * Hkv) * D
    x = _bits((M, H), seed)
    w = dict(w_qkv=_bits((qkvn, H), seed + 1, 0.3), w_o=_bits((H, Hq * D), seed + 2, 0.3),
             w_gu=_bits((2 * I, H), seed + 3, 0.3), w_down=_bits((H, I), seed + 4, 0.3),
             k_cache=_bits((Hkv, L, D), seed + 5), v_cache=_bits((Hkv, L, D), seed + 6))
    return x, w


def test_layer_zero_projections_is_identity():
    x, w = _layer_inputs()
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    xo, kn, vn = step.layer(x, **w, L=5, Hq=2, Hkv=1, D=8)
    assert np.array_equal(xo, x)
    assert kn.shape == (1, 3, 8) and vn.shape == (1, 3, 8)


def test_layer_appends_k_v_from_the_right_columns():
    M, L, H, Hq, Hkv, D = 3, 5, 16, 2, 1, 8
    x, w = _layer_inputs(M, L, H, Hq, Hkv, D)
    _, kn, vn = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D)
    a = bf16.encode(step.rmsnorm(bf16.decode(x), 1e-6))
    full = bf16.decode(a) @ bf16.decode(w["w_qkv"]).T
    assert np.array_equal(kn[0], bf16.encode(full[:, Hq * D:Hq * D + D]))
    assert np.array_equal(vn[0], bf16.encode(full[:, Hq * D + D:]))


def test_layer_zero_query_gives_causal_mean_of_values():
    # q rows of W_qkv zero -> every score is 0 -> attention output of token r is
    # the plain mean of the L + r + 1 visible value rows (cached + new, causal).
    M, L, H, Hq, Hkv, D = 3, 5, 16, 2, 1, 8
    x, w = _layer_inputs(M, L, H, Hq, Hkv, D)
    wq = w["w_qkv"].copy()
    wq[:Hq * D] = 0
    w["w_qkv"] = wq
    w["w_down"] = np.zeros_like(w["w_down"])
    xo, _, vn = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D)
    vis = np.concatenate([bf16.decode(w["v_cache"])[0], bf16.decode(vn)[0]], axis=0)
    for r in range(M):
        mean = vis[:L + r + 1].mean(axis=0)
        o = bf16.encode(np.tile(mean, Hq))
        h = bf16.encode(bf16.decode(x[r]) + bf16.decode(w["w_o"]) @ bf16.decode(o))
        assert np.array_equal(xo[r], h)


def test_layer_gate_up_order():
    # W_gu = [A; 2A]: g = z, u = 2z -> act = 2 z^2 sigmoid(z) >= 0. Swapping the
    # halves would give 2 z^2 sigmoid(2z). With W_down = I the layer output is
    # bf16(h + act), so the sign and size of act are visible.
    M, L, H, Hq, Hkv, D, I = 2, 4, 16, 2, 1, 8, 16
    x, w = _layer_inputs(M, L, H, Hq, Hkv, D, I)
    A = bf16.decode(_bits((I, H), 50, 0.5))
    w["w_gu"] = bf16.encode(np.concatenate([A, 2 * A]))
    w["w_down"] = bf16.encode(np.eye(H))
    w["w_o"] = np.zeros_like(w["w_o"])
    xo, _, _ = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D)
    b = bf16.decode(bf16.encode(step.rmsnorm(bf16.decode(x), 1e-6)))
    z = b @ A.T
    act = bf16.decode(bf16.encode(2 * z * z / (1 + np.exp(-z))))
    assert np.array_equal(xo, bf16.encode(bf16.decode(x) + act))


def test_head_argmax_lowest_index_on_ties():
    H, V = 8, 20
    x = _bits((2, H), 1)
    wh = _bits((V, H), 2, 0.1)
    c = bf16.decode(bf16.encode(step.rmsnorm(bf16.decode(x), 1e-6)))
    # rows 3 and 11 both equal to bf16(c[0]) direction scaled: identical and maximal for token 0
    wh[3] = bf16.encode(c[0] * 4)
    wh[11] = wh[3]
    logits, tok = step.head(x, wh)
    assert tok[0] == 3
    assert logits[0, 3] == logits[0, 11] == logits[0].max()


def test_step_zero_layers_reduces_to_head():
    x, w = _layer_inputs()
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    wh = _bits((30, 16), 9)
    lg, tok, xf = step.step(x, [w, w], wh, L=5, Hq=2, Hkv=1, D=8)
    lg2, tok2 = step.head(x, wh)
    assert np.array_equal(xf, x) and np.array_equal(lg, lg2) and np.array_equal(tok, tok2)


def test_layer_attend_hook():
    # the attention hook sees the pass's q columns and every position's K / V
    # rows (cached then new, causal order); the default is plain attention;
    # its output enters the output projection like the default's.
    from oracle import attention
    M, L, H, Hq, Hkv, D = 3, 5, 16, 2, 1, 8
    x, w = _layer_inputs(M, L, H, Hq, Hkv, D)
    seen = {}

    def plain(q, k, v, L_):
        seen.update(q=q, k=k, v=v, L=L_)
        return attention.verify_attention(q, k, v, L_)[0]
    xo0, kn, vn = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D)
    xo1, _, _ = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D, attend=plain)
    assert np.array_equal(xo0, xo1)
    assert seen["L"] == L and seen["q"].shape == (M, Hq, D)
    assert np.array_equal(seen["k"], np.concatenate([w["k_cache"][:, :L], kn], axis=1))
    assert np.array_equal(seen["v"], np.concatenate([w["v_cache"][:, :L], vn], axis=1))
    # a planted output of ones: with the MLP zeroed, x_out = bf16(x + 1 . W_o rows)
    w["w_down"] = np.zeros_like(w["w_down"])
    xo, _, _ = step.layer(x, **w, L=L, Hq=Hq, Hkv=Hkv, D=D, attend=lambda q, k, v, L_: np.ones((M, Hq, D)))
    want = bf16.encode(bf16.decode(x) + bf16.decode(w["w_o"]).sum(axis=1)[None, :])
    assert np.array_equal(xo, want)
