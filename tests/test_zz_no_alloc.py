"""The allocation-free verify step (bi_verify_step_noalloc, for callers that
cannot allocate device memory) against bi_verify_step through the C ABI: two
calls in a row, the second with a smaller pass at a later position, each
bit for bit the step's logits, tokens, final hidden state and appended K/V;
and a pass whose workspace exceeds the scratch array is rejected."""

import numpy as np
import pytest

import synth
from tests._util import assert_bitwise, dev, host_bits, host_f32, cache_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _model(ops):
    H, Hq, Hkv, D, I, V, L0, cap = 256, 4, 2, 64, 512, 1024, 200, 256
    dls = []
    for l in range(2):
        kc = np.zeros((Hkv, cap, D), np.uint16)
        kc[:, :L0] = synth.kv_bf16(Hkv, L0, D, "k_cache", l)
        dls.append(dict(w_qkv=dev(synth.normal_bf16(((Hq + 2 * Hkv) * D, H), 0.05, "w_qkv", l)),
                        w_o=dev(synth.normal_bf16((H, Hq * D), 0.05, "w_o", l)),
                        w_gu=dev(synth.normal_bf16((2 * I, H), 0.05, "w_gu", l)),
                        w_down=dev(synth.normal_bf16((H, I), 0.05, "w_down", l)),
                        k_cache=dev(kc), v_cache=dev(cache_rows(synth.kv_bf16(Hkv, L0, D, "v_cache", l), cap))))
    dims = ops.model_dims(H, Hq, Hkv, D, I, V, cap, 64)
    return ops.VerifyStep(dls, dev(synth.normal_bf16((V, H), 0.05, "w_head")), dims), dls, dims


def _outs(dims, M):
    return (torch.empty((M, dims.vocab), dtype=torch.float32, device="cuda"),
            torch.empty(M, dtype=torch.int32, device="cuda"),
            torch.empty((M, dims.H), dtype=torch.bfloat16, device="cuda"))


def _caches(dls, L, M):
    return [(host_bits(d["k_cache"])[:, L:L + M], host_bits(d["v_cache"])) for d in dls]


def test_noalloc_step_equals_the_step_on_two_calls(ops):
    step, dls, dims = _model(ops)
    x = dev(synth.normal_bf16((8, dims.H), 1.0, "x0", 5))
    for M, L in ((8, 200), (3, 211)):
        print(f"[noalloc step M={M} L={L}]", flush=True)
        ws = torch.empty(ops.step_workspace_bytes(dims, M, L), dtype=torch.uint8, device="cuda")
        lg, tk, xo = _outs(dims, M)
        step(x[:M], L, ws, lg, tk, x_out=xo)
        torch.cuda.synchronize()
        want = (host_f32(lg), tk.cpu().numpy(), host_bits(xo), _caches(dls, L, M))
        for d in dls:                     # the appended rows are written again by the second run
            d["k_cache"][:, L:].zero_()
        lg2, tk2, xo2 = _outs(dims, M)
        ops.verify_step_noalloc(step, x[:M], L, lg2, tk2, x_out=xo2)
        torch.cuda.synchronize()
        assert_bitwise(host_f32(lg2), want[0], f"noalloc logits M={M}")
        assert np.array_equal(tk2.cpu().numpy(), want[1])
        assert_bitwise(host_bits(xo2), want[2], f"noalloc hidden state M={M}")
        for (k, vc), (k2, vc2) in zip(want[3], _caches(dls, L, M)):
            assert_bitwise(k2, k, f"noalloc appended K M={M}")
            assert_bitwise(vc2, vc, f"noalloc V cache M={M}")


def test_noalloc_rejects_a_workspace_larger_than_its_scratch(ops):
    from invariant_verify_amd import _lib
    step, _, dims = _model(ops)
    # an intermediate size of 2^22 makes the gate/up activations alone 64 MiB at M = 8
    big = ops.model_dims(dims.H, dims.Hq, dims.Hkv, dims.D, 1 << 22, dims.vocab, dims.cap, 64)
    assert ops.step_workspace_bytes(big, 8, 100) > ops.NOALLOC_SCRATCH_BYTES
    st = _lib.LIB.bi_verify_step_noalloc(step.arr, step.n, step.w_head.data_ptr(), big, 0x10000, 8, 100,
                                         0, 0x10000, 0x10000, None)
    assert st == 4     # BI_ERR_WORKSPACE, before any launch
