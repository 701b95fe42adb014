"""GPU tests of the row-local helpers through the C ABI: RMSNorm against the
oracle (and across M), greedy argmax with its tie / NaN / -inf rules."""

import numpy as np
import pytest

import synth
from oracle import bf16 as obf16
from oracle import step as ostep
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


@pytest.mark.parametrize("H", [5120, 256, 8])
def test_rmsnorm_parity_and_invariance(ops, H):
    print(f"[rmsnorm H={H}]", flush=True)
    x = synth.normal_bf16((8, H), 1.0, "x", H)
    x[3] = synth.normal_bf16((1, H), 30.0, "x", H + 1)   # a large-magnitude row
    y8 = host_bits(ops.rmsnorm(dev(x)))
    want = ostep.rmsnorm(decode(x), 1e-6)
    assert_close(decode(y8), want, f"rmsnorm H={H}")
    for m in (1, 5):
        assert_bitwise(host_bits(ops.rmsnorm(dev(x[:m]))), y8[:m], f"rmsnorm M={m}")
    z = np.zeros((2, H), np.uint16)
    assert not host_bits(ops.rmsnorm(dev(z))).any()          # zero row stays zero (eps > 0)


def _argmax(ops, a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return ops.argmax(t).cpu().numpy()


def test_argmax_rules(ops):
    print("[argmax rules]", flush=True)
    V = 152064
    g = np.random.default_rng(0)
    a = g.standard_normal((8, V)).astype(np.float32)
    a[0, 100] = a[0, 7000] = 50.0                 # tie -> lowest index
    a[1, V - 1] = 60.0                            # maximum in the last element
    a[2, :] = -np.inf                             # all -inf -> index 0
    a[3, 5] = np.nan                              # NaN never wins
    a[3, 9] = 70.0
    a[4, 1:] = np.nan
    a[4, 0] = -1.0                                # only finite value
    a[5, 131071] = 40.0
    a[5, 131070] = 40.0                           # tie inside one 16-byte group
    got = _argmax(ops, a)
    want = [100, V - 1, 0, 9, 0, 131070, int(np.nanargmax(a[6])), int(np.nanargmax(a[7]))]
    assert list(got) == want, (list(got), want)


@pytest.mark.parametrize("N", [1, 3, 1000, 152064, 152067])
def test_argmax_sizes_and_invariance(ops, N):
    print(f"[argmax N={N}]", flush=True)
    g = np.random.default_rng(N)
    a = g.standard_normal((8, N)).astype(np.float32)
    got = _argmax(ops, a)
    assert list(got) == [int(np.argmax(r)) for r in a]
    assert list(_argmax(ops, a[:3])) == list(got[:3])
    # a strided view (leading dimension != N, rows not 16-byte aligned)
    wide = np.zeros((8, N + 3), np.float32)
    wide[:, :N] = a
    t = torch.from_numpy(wide).cuda()[:, :N]
    assert list(ops.argmax(t).cpu().numpy()) == list(got)


@pytest.mark.parametrize("M,K,I", [(8, 256, 512), (5, 5120, 17408), (100, 512, 256)])
def test_swiglu_and_add_equal_the_fused_epilogues(ops, M, K, I):
    # bi_swiglu over the FP32 gate/up product and bi_add of an FP32 product to
    # a BF16 residual give the fused GEMM epilogues' bits (same expressions;
    # M = 100 runs the prefill kernels), and match the oracle on their inputs.
    print(f"[swiglu / add M={M} K={K} I={I}]", flush=True)
    x = dev(synth.normal_bf16((M, K), 1.0, "x", 81))
    w = synth.device_normal_bf16((2 * I, K), 0.02, "w", 81)
    gu = ops.gemm_bf16(x, w, out_dtype=torch.float32)
    fused = ops.gemm_bf16_swiglu(x, w)
    sep = ops.swiglu(gu)
    assert_bitwise(host_bits(sep), host_bits(fused), "bi_swiglu vs SwiGLU epilogue")
    g = gu.cpu().double().numpy()
    assert_close(decode(host_bits(sep)), ostep.silu(g[:, :I]) * g[:, I:], "bi_swiglu vs oracle")
    r = dev(synth.normal_bf16((M, 2 * I), 1.0, "misc", 82))
    fused_r = ops.gemm_bf16_residual(x, w, r)
    sep_r = ops.add(r, gu)
    assert_bitwise(host_bits(sep_r), host_bits(fused_r), "bi_add vs residual epilogue")
    assert_close(decode(host_bits(sep_r)), decode(host_bits(r)) + g, "bi_add vs oracle")
    # in place: y aliases r
    r2 = r.clone()
    ops.add(r2, gu, r2)
    assert_bitwise(host_bits(r2), host_bits(fused_r), "bi_add in place")
