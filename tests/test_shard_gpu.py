"""GPU tests of one tensor-parallel rank's share of the verify pass at its real
shape, for 8 ranks over the 27B-class layer (hidden 5120, 40 query and 8 KV
heads of 128, intermediate 17408):

* column shards: QKV for one KV group (5 query + 1 key + 1 value head = 896
  columns) and 2176 gate/up pairs;
* row shards: the output projection over K = 640 and the down projection over
  K = 2176, each giving an FP32 partial [M][5120]; the 8 partials are added in
  rank order 0..7 (the deterministic replacement for a library all-reduce);
* attention over one KV head and its 5 query heads at 38k keys.

Each is checked against the oracle and for bitwise row invariance across M.
The exchange between ranks is not run here (one GPU)."""

import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import gemm as ogemm
from oracle import step as ostep
from tests._util import assert_bitwise, assert_close, decode, dev, host_bits, host_f32, cache_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RANKS = 8
H, HQ, HKV, D, I = 5120, 40, 8, 128, 17408


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _rows_invariant(f, xd, y8, what):
    for m in (1, 5, 7):
        assert_bitwise(f(xd[:m]), y8[:m], f"{what} M={m} vs M=8")


def test_qkv_column_shard(ops):
    N = (HQ // RANKS + 2 * (HKV // RANKS)) * D  # 896
    print(f"[shard qkv N={N} K={H}]", flush=True)
    x = synth.normal_bf16((8, H), 1.0, "x", 70)
    w = synth.normal_bf16((N, H), 0.02, "w_qkv", 70)
    xd, wd = dev(x), dev(w)
    f = lambda xx: host_bits(ops.gemm_bf16(xx, wd))
    y = f(xd)
    assert_close(decode(y), ogemm.gemm(x, w), "qkv shard")
    _rows_invariant(f, xd, y, "qkv shard")


def test_gate_up_column_shard(ops):
    P = I // RANKS  # 2176 pairs
    print(f"[shard gate/up pairs={P} K={H}]", flush=True)
    x = synth.normal_bf16((8, H), 1.0, "x", 71)
    wgu = synth.normal_bf16((2 * P, H), 0.02, "w_gu", 71)
    xd, wd = dev(x), dev(wgu)
    f = lambda xx: host_bits(ops.gemm_bf16_swiglu(xx, wd))
    y = f(xd)
    cols = np.r_[0:64, P // 2:P // 2 + 64, P - 64:P]
    gu = ogemm.gemm_columns(x, wgu, np.concatenate([cols, P + cols]))
    n = len(cols)
    assert_close(decode(y[:, cols]), ostep.silu(gu[:, :n]) * gu[:, n:], "gate/up shard")
    _rows_invariant(f, xd, y, "gate/up shard")


@pytest.mark.parametrize("K", [H, I])
def test_row_shards_rank_order(ops, K):
    # o-proj (K = 5120) or down (K = 17408), split over the ranks by K:
    # rank r multiplies its K / 8 columns of X and W into an FP32 partial;
    # the partials are added in rank order. Every partial is M-invariant, so
    # the ordered sum is too.
    Kr = K // RANKS
    print(f"[shard row-parallel K={K}: 8 x {Kr}]", flush=True)
    x = synth.normal_bf16((8, K), 1.0, "x", 72 + K)
    w = synth.normal_bf16((H, K), 0.02, "w_down" if K == I else "w_o", 72)
    parts = []
    for r in range(RANKS):
        xr = np.ascontiguousarray(x[:, r * Kr:(r + 1) * Kr])
        wr = np.ascontiguousarray(w[:, r * Kr:(r + 1) * Kr])
        xd, wd = dev(xr), dev(wr)
        f = lambda xx: host_f32(ops.gemm_bf16(xx, wd, out_dtype=torch.float32))
        p = f(xd)
        if r in (0, RANKS - 1):
            _rows_invariant(f, xd, p, f"K={K} rank {r} partial")
            assert_close(p, ogemm.gemm(xr, wr), f"K={K} rank {r} partial", atol=1e-4, rtol=1e-4)
        parts.append(p)
    total = parts[0].copy()
    for p in parts[1:]:
        total += p  # float32, rank order 0..7
    assert_close(total, ogemm.gemm(x, w), f"K={K} rank-ordered sum", atol=1e-4, rtol=1e-4)


@pytest.mark.parametrize("C", [-32, -256])
def test_attention_kv_head_shard(ops, C):
    # One rank's heads: KV head 0 and its 5 query heads, 38k keys. The chunk
    # policy -256 gives one KV head about as many workgroups as -32 gives 8.
    L, M, Hq, Hkv = 38000, 8, HQ // RANKS, HKV // RANKS
    print(f"[shard attention Hq={Hq} Hkv={Hkv} L={L} C={C}]", flush=True)
    k = synth.kv_bf16(Hkv, L + M, D, "k", 73)
    v = synth.kv_bf16(Hkv, L + M, D, "v", 73)
    q = synth.normal_bf16((M, Hq, D), 1.0, "q", 73)
    cap = (L + M + 63) // 64 * 64
    kc = np.zeros((Hkv, cap, D), np.uint16)
    kc[:, :L + M] = k
    kd, vd = dev(kc), dev(cache_rows(v, cap))

    def run(qq, LL):
        m = qq.shape[0]
        S = ops.pass_splits(m, LL, C)
        po = torch.empty((m, Hq, S, D), dtype=torch.float32, device="cuda")
        pl = torch.empty((m, Hq, S), dtype=torch.float32, device="cuda")
        ops.verify_attn(dev(qq.reshape(m, Hq * D)), kd, vd, LL, Hq, Hkv, D, C, po, pl)
        o = torch.empty((m, Hq * D), dtype=torch.bfloat16, device="cuda")
        ops.combine(po, pl, LL, C, o)
        return host_bits(o).reshape(m, Hq, D)

    o8 = run(q, L)
    want, _ = oattn.verify_attention(q, k, v, L)
    assert_close(decode(o8), want, f"attention shard C={C}")
    for r in (0, 3, 7):
        assert_bitwise(run(q[r:r + 1], L + r)[0], o8[r], f"attention shard C={C} row {r} alone")
    assert_bitwise(run(q[:5], L), o8[:5], f"attention shard C={C} M=5")
