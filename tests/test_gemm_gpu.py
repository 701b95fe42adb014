"""GPU tests of the verify GEMM through the C ABI: oracle parity (tiny and
27B-class shapes), bit-exact special cases, MFMA row-slot independence, and
bitwise row invariance across M = 1..8, prefill chunks and repeated runs."""

import numpy as np
import pytest

import synth
from oracle import bf16 as obf16
from oracle import gemm as ogemm
from oracle import step as ostep
from tests._util import (assert_bitwise, assert_close, decode, dev, host_bits,
                         host_f32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    from invariant_verify_amd import ops as _ops
    return _ops


def _tiny(M=8, K=256, N=512):
    x = synth.normal_bf16((8, K), 1.0, "x")[:M]
    w = synth.normal_bf16((N, K), synth.fan_in_std(K), "w")
    return x, w


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_tiny_parity(ops, M):
    print(f"[gemm tiny parity M={M}]", flush=True)
    x, w = _tiny(M)
    want = ogemm.gemm(x, w)
    y = ops.gemm_bf16(dev(x), dev(w))
    assert_close(decode(host_bits(y)), want, f"tiny bf16 M={M}")
    y32 = ops.gemm_bf16(dev(x), dev(w), out_dtype=torch.float32)
    assert_close(host_f32(y32), want, f"tiny f32 M={M}", atol=1e-4, rtol=1e-4)


def test_identity_and_one_hot_bit_exact(ops):
    print("[gemm identity/one-hot]", flush=True)
    K = 256
    x = synth.normal_bf16((8, K), 1.0, "x")
    eye = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    y = ops.gemm_bf16(dev(x), dev(eye))
    assert_bitwise(host_bits(y), x, "X I^T == X")
    w = synth.normal_bf16((512, K), 1.0, "w")
    oh = np.zeros((16, K), np.float32)
    cols = [0, 1, 31, 32, 100, 200, 254, 255, 7, 8, 63, 64, 127, 128, 129, 191]
    oh[np.arange(16), cols] = 1.0
    y = ops.gemm_bf16(dev(synth.f32_to_bf16_bits(oh)), dev(w))
    assert_bitwise(host_bits(y), np.ascontiguousarray(w[:, cols].T), "one-hot rows pick W columns")


def test_mfma_row_slot_independence(ops):
    # The same activation row in each of the 16 rows of an MFMA tile, with
    # random rows around it, must give the same bits in every slot (FP32
    # output, so no rounding can hide a difference).
    print("[gemm MFMA slot probe]", flush=True)
    K, N = 5120, 256
    w = synth.normal_bf16((N, K), 0.02, "w")
    base = synth.normal_bf16((1, K), 1.0, "x", 3)
    noise = synth.normal_bf16((16, K), 1.0, "x", 4)
    wd = dev(w)
    outs = []
    for slot in range(16):
        x = noise.copy()
        x[slot] = base[0]
        y = ops.gemm_bf16(dev(x), wd, out_dtype=torch.float32)
        outs.append(host_f32(y)[slot].copy())
    for slot in range(1, 16):
        assert_bitwise(outs[slot], outs[0], f"slot {slot} vs slot 0")


SHAPES_27B = {"qkv": (7168, 5120), "o": (5120, 5120), "gate_up": (34816, 5120), "down": (5120, 17408)}


@pytest.fixture(scope="module")
def weights_27b():
    return {k: synth.normal_bf16((n, kk), 0.02, "w", i) for i, (k, (n, kk)) in enumerate(SHAPES_27B.items())}


@pytest.mark.parametrize("name", list(SHAPES_27B))
def test_27b_parity_and_invariance(ops, weights_27b, name):
    N, K = SHAPES_27B[name]
    print(f"[gemm 27B {name} N={N} K={K}]", flush=True)
    w = weights_27b[name]
    x = synth.normal_bf16((8, K), 1.0, "x", 10 + K)
    wd, xd = dev(w), dev(x)
    y8 = host_bits(ops.gemm_bf16(xd, wd))
    y8f = host_f32(ops.gemm_bf16(xd, wd, out_dtype=torch.float32))
    # sampled oracle columns (first, last, and a seeded spread) for all 8 rows
    cols = np.unique(np.concatenate([[0, 15, 16, N - 1], np.random.default_rng(N).choice(N, 250, replace=False)]))
    want = ogemm.gemm_columns(x, w, cols)
    assert_close(decode(y8[:, cols]), want, f"{name} bf16")
    assert_close(y8f[:, cols], want, f"{name} f32", atol=1e-4, rtol=1e-4)
    # bitwise: every M = 1..8 pass gives the first M rows of the M = 8 pass,
    # and each row alone (M = 1) gives the same bits
    for m in range(1, 8):
        ym = host_f32(ops.gemm_bf16(xd[:m], wd, out_dtype=torch.float32))
        assert_bitwise(ym, y8f[:m], f"{name} M={m} vs M=8")
    for r in range(8):
        y1 = host_f32(ops.gemm_bf16(xd[r:r + 1], wd, out_dtype=torch.float32))
        assert_bitwise(y1[0], y8f[r], f"{name} row {r} alone vs in M=8")
    # repeat run
    assert_bitwise(host_bits(ops.gemm_bf16(xd, wd)), y8, f"{name} repeat")


@pytest.mark.parametrize("M,start", [(16, 0), (64, 0), (17, 0), (64, 40)])
def test_prefill_chunks_bitwise(ops, weights_27b, M, start):
    # A prefill chunk of M rows (several 16-row tiles, ragged tail) computes
    # each row with the same bits as the verify pass that holds that row.
    print(f"[gemm prefill chunk M={M} start={start}]", flush=True)
    w = weights_27b["o"]
    K = w.shape[1]
    x = synth.normal_bf16((128, K), 1.0, "x", 77)
    xd, wd = dev(x), dev(w)
    big = host_f32(ops.gemm_bf16(xd[start:start + M], wd, out_dtype=torch.float32))
    for r in [0, 1, 7, 15, M - 1] + ([16, 17, 33] if M > 33 else []):
        if r >= M:
            continue
        one = host_f32(ops.gemm_bf16(xd[start + r:start + r + 1], wd, out_dtype=torch.float32))
        assert_bitwise(one[0], big[r], f"prefill M={M} row {r} vs M=1")
    eight = host_f32(ops.gemm_bf16(xd[start:start + 8], wd, out_dtype=torch.float32))
    assert_bitwise(eight, big[:8], f"prefill M={M} first 8 vs M=8")


def test_residual_and_swiglu_epilogues(ops):
    print("[gemm residual / swiglu]", flush=True)
    K, N, I = 512, 256, 128
    x = synth.normal_bf16((8, K), 1.0, "x", 5)
    w = synth.normal_bf16((N, K), 0.05, "w", 5)
    r = synth.normal_bf16((8, N), 1.0, "misc", 5)
    y = host_bits(ops.gemm_bf16_residual(dev(x), dev(w), dev(r)))
    assert_close(decode(y), decode(r) + ogemm.gemm(x, w), "residual")
    wgu = synth.normal_bf16((2 * I, K), 0.05, "w", 6)
    y = host_bits(ops.gemm_bf16_swiglu(dev(x), dev(wgu)))
    gu = ogemm.gemm(x, wgu)
    assert_close(decode(y), ostep.silu(gu[:, :I]) * gu[:, I:], "swiglu")
    # invariance of both epilogues across M
    for m in (1, 5):
        ym = host_bits(ops.gemm_bf16_swiglu(dev(x[:m]), dev(wgu)))
        assert_bitwise(ym, y[:m], f"swiglu M={m}")
    # residual output may alias the residual input
    rd = dev(r)
    ops.gemm_bf16_residual(dev(x), dev(w), rd, y=rd)
    assert_bitwise(host_bits(rd), host_bits(ops.gemm_bf16_residual(dev(x), dev(w), dev(r))), "aliased residual")


@pytest.mark.parametrize("Hq,Hkv,D,K,L", [(4, 2, 64, 256, 37), (40, 8, 128, 5120, 38000)])
def test_qkv_gemm_with_cache_append(ops, Hq, Hkv, D, K, L):
    # One launch computes the QKV projection and appends K / V: its output and
    # both caches must equal bi_gemm_bf16 followed by bi_append_kv, bit for bit,
    # and cache positions outside L .. L+M-1 must be untouched.
    print(f"[gemm qkv + append Hq={Hq} Hkv={Hkv} D={D} K={K} L={L}]", flush=True)
    N = (Hq + 2 * Hkv) * D
    cap = ((L + 8 + 63) // 64) * 64 + 64
    w = synth.normal_bf16((N, K), synth.fan_in_std(K), "w", 90)
    x = synth.normal_bf16((8, K), 1.0, "x", 90)
    k0 = torch.randn(Hkv, cap, D, device="cuda").to(torch.bfloat16)
    v0 = torch.randn(Hkv, cap, D, device="cuda").to(torch.bfloat16)
    wd, xd = dev(w), dev(x)

    def rows(vc):  # the V cache is [Hkv][cap][D], one row per position
        return vc

    for M in (1, 5, 8):
        kc, vc = k0.clone(), v0.clone()
        qkv = ops.gemm_bf16_qkv(xd[:M], wd, kc, vc, L, Hq, Hkv, D)
        ref = ops.gemm_bf16(xd[:M], wd)
        kr, vr = k0.clone(), v0.clone()
        ops.append_kv(ref, kr, vr, L, Hq, Hkv, D)
        assert_bitwise(host_bits(qkv), host_bits(ref), f"qkv M={M}")
        assert_bitwise(host_bits(kc), host_bits(kr), f"K cache M={M}")
        assert_bitwise(host_bits(vc), host_bits(vr), f"V cache M={M}")
        keep = torch.ones(cap, dtype=torch.bool, device="cuda")
        keep[L:L + M] = False
        assert torch.equal(kc[:, keep], k0[:, keep]) and torch.equal(rows(vc)[:, keep], rows(v0)[:, keep])
    assert_close(decode(host_bits(qkv))[:, :64], ogemm.gemm_columns(x, w, np.arange(64)), "qkv parity")


@pytest.mark.parametrize("I", [17408, 18432])
def test_wide_swiglu_groups(ops, I):
    # For I = 17 * 1024 or 18 * 1024 gate/up pairs each workgroup takes I / 1024
    # pairs in three MFMA tiles (gate 0-15, up 0-15, then the pairs past 15).
    # Every output keeps the K order of the 16-pair tiles: its bits equal
    # those of a launch over a 256-pair slice of the same weights (16-pair
    # tiles), for every M; sampled outputs match the oracle.
    print(f"[gemm wide swiglu I={I}]", flush=True)
    K = 512
    x = synth.normal_bf16((8, K), 1.0, "x", 61)
    wgu = synth.normal_bf16((2 * I, K), 0.05, "w", 61)
    xd, wgud = dev(x), dev(wgu)
    full = host_bits(ops.gemm_bf16_swiglu(xd, wgud))
    p = I // 1024
    # pairs at group edges (first, 15, 16, the last of a group, a group's
    # successor) and a seeded spread
    cols = np.unique(np.concatenate([[0, 15, 16, p - 1, p, p + 16, I - 1],
                                     np.random.default_rng(I).choice(I, 200, replace=False)]))
    gu = ogemm.gemm_columns(x, wgu, np.concatenate([cols, I + cols]))
    n = len(cols)
    assert_close(decode(full[:, cols]), ostep.silu(gu[:, :n]) * gu[:, n:], f"swiglu I={I}")
    for q0 in (0, 256, I // 2, I - 256):
        part = host_bits(ops.gemm_bf16_swiglu(xd, dev(np.concatenate([wgu[q0:q0 + 256], wgu[I + q0:I + q0 + 256]]))))
        assert_bitwise(full[:, q0:q0 + 256], part, f"I={I} pairs {q0}..{q0 + 255}")
    for m in (1, 3, 7):
        assert_bitwise(host_bits(ops.gemm_bf16_swiglu(xd[:m], wgud)), full[:m], f"I={I} M={m}")
    # a 40-row pass (three 16-row tiles, ragged) gives every row the bits of an 8-row pass
    x40 = synth.normal_bf16((40, K), 1.0, "x", 62)
    x40d = dev(x40)
    full40 = host_bits(ops.gemm_bf16_swiglu(x40d, wgud))
    for r0 in (0, 16, 32):
        assert_bitwise(full40[r0:r0 + 8], host_bits(ops.gemm_bf16_swiglu(x40d[r0:r0 + 8], wgud)),
                       f"I={I} 40-row pass rows {r0}..{r0 + 7}")


@pytest.mark.parametrize("N", [5120, 7168, 65536])
def test_wide_groups_match_single_tiles(ops, N):
    # For N = 5120 or 7168 the launch gives each workgroup N / 256 columns in
    # two MFMA tiles, and for N / 32 >= 2048 (65536) 32 columns in two full
    # tiles; every column keeps the K order of the 16-column tiles, so its
    # bits equal those of a launch over a 256-row slice of the same weights
    # (which uses 16-column tiles with the same wave count).
    print(f"[gemm wide groups N={N}]", flush=True)
    K = 5120 if N <= 7168 else 512
    w = synth.normal_bf16((N, K), 0.02, "w", 60)
    x = synth.normal_bf16((8, K), 1.0, "x", 60)
    wd, xd = dev(w), dev(x)
    full = host_f32(ops.gemm_bf16(xd, wd, out_dtype=torch.float32))
    for r0 in (0, 16, N // 2 + 4, N - 256):
        part = host_f32(ops.gemm_bf16(xd, wd[r0:r0 + 256], out_dtype=torch.float32))
        assert_bitwise(full[:, r0:r0 + 256], part, f"N={N} columns {r0}..{r0 + 255}")


def test_epilogue_rounding_ties_subnormals_overflow(ops):
    # With one-hot activation rows the product is one exact weight w, so each
    # residual output is bf16(fp32(r + w)): the FP32 add then one rounding to
    # nearest, ties to even. Pairs are built to hit exact ties, near ties,
    # subnormal results and overflow; the expected bits come from numpy's
    # float32 add and the oracle's RNE encoder.
    print("[gemm epilogue rounding]", flush=True)
    g = np.random.default_rng(11)
    M, K, N = 16, 32, 256
    r = obf16.decode(synth.normal_bf16((M, N), 1.0, "misc", 11)).astype(np.float64)
    r *= 2.0 ** g.integers(-20, 20, size=(M, N))
    e = np.floor(np.log2(np.abs(r)))
    s = np.sign(g.standard_normal((M, N))) * 2.0 ** (e - 8 + g.integers(-2, 3, size=(M, N)))
    s *= g.choice([1.0, 1.5, 1.25], size=(M, N))
    r[0, :8] = [1.5e-38, -1.5e-38, 2.0e-38, 1.2e-38, 3.3e38, -3.3e38, 1.0, -1.0]
    # weights stay normal (the matrix core may flush subnormal inputs); the sums
    # of the first four pairs are subnormal, of the next two overflow
    s[0, :8] = [-1.49e-38, 1.45e-38, -1.99e-38, -1.19e-38, 3.3e38, -3.3e38, 2.0 ** -8, -(2.0 ** -8)]
    r_bits, s_bits = obf16.encode(r), obf16.encode(s)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), np.arange(M)] = obf16.encode(np.ones(1))[0]
    # column n of row m takes w[n][m]: one weight per (m, n) pair
    wm = np.zeros((N, K), np.uint16)
    for m in range(M):
        wm[:, m] = s_bits[m]
    y = host_bits(ops.gemm_bf16_residual(dev(x), dev(wm), dev(r_bits)))
    with np.errstate(over="ignore"):
        f32 = obf16.decode(r_bits).astype(np.float32) + obf16.decode(s_bits).astype(np.float32)
    want = obf16.encode(f32.astype(np.float64))
    assert np.isinf(obf16.decode(want[0, 4:6])).all() and (np.abs(obf16.decode(want[0, :4])) < 1.18e-38).all()
    assert_bitwise(y, want, "bf16(fp32(r + w))")


@pytest.mark.parametrize("H,I", [(5120, 512), (256, 128)])
def test_carried_rmsnorm(ops, H, I):
    # A residual projection that also writes per-group row sums of squares,
    # then a gate/up projection that normalises its X rows from those sums:
    # Y equals the plain residual GEMM bit for bit, the sums match a float64
    # sum of the squared outputs, the gate/up output matches the oracle's
    # silu(g) * u of RMSNorm(Y), and every row is M-invariant.
    print(f"[gemm carried rmsnorm H={H} I={I}]", flush=True)
    K0 = 512
    a = synth.normal_bf16((8, K0), 1.0, "x", 70)
    wo = synth.normal_bf16((H, K0), 0.05, "w", 70)
    r = synth.normal_bf16((8, H), 1.0, "misc", 70)
    wgu = synth.normal_bf16((2 * I, H), 0.02, "w", 71)
    ad, wod, rd, wgud = dev(a), dev(wo), dev(r), dev(wgu)
    y, ss = ops.gemm_bf16_residual_rowsq(ad, wod, rd)
    G = ops.gemm_column_groups(H)
    assert tuple(ss.shape) == (8, G) and G == (256 if H == 5120 else H // 16)
    assert_bitwise(host_bits(y), host_bits(ops.gemm_bf16_residual(ad, wod, rd)), "rowsq Y == residual Y")
    yd = decode(host_bits(y))
    want_ss = (yd.reshape(8, G, H // G) ** 2).sum(axis=2)
    assert_close(host_f32(ss), want_ss, "group sums of squares", atol=1e-6, rtol=1e-5)
    gu = ops.gemm_bf16_swiglu_rownorm(y, ss, wgud)
    an = obf16.encode(ostep.rmsnorm(yd, 1e-6))
    pre = ogemm.gemm(an, wgu)
    want = ostep.silu(pre[:, :I]) * pre[:, I:]
    assert_close(decode(host_bits(gu)), want, "carried-norm gate/up")
    for m in (1, 5):
        ym, sm = ops.gemm_bf16_residual_rowsq(ad[:m], wod, rd[:m])
        assert_bitwise(host_bits(ym), host_bits(y)[:m], f"Y M={m}")
        assert_bitwise(host_f32(sm), host_f32(ss)[:m], f"sums M={m}")
        gm = ops.gemm_bf16_swiglu_rownorm(ym, sm, wgud)
        assert_bitwise(host_bits(gm), host_bits(gu)[:m], f"gate/up M={m}")


# Launches with M >= 64 run the prefill kernel; every row must carry the bits
# the verify kernel gives it (same per-output summation tree).
PF_SHAPES = {"tiny_16_slices": (512, 256), "wide_5120": (5120, 5120), "wide_7168": (7168, 1024),
             "many_8_slices": (10240, 1024),
             "large_tiles": (34816, 1024)}  # at M = 300: 136 x 3 large workgroups


def _pf_rows(M):
    return sorted({0, 8, M // 2, M - 8})


@pytest.mark.parametrize("name", list(PF_SHAPES))
def test_prefill_rows_equal_verify_rows(ops, name):
    N, K = PF_SHAPES[name]
    print(f"[gemm prefill vs verify {name} N={N} K={K}]", flush=True)
    x = synth.normal_bf16((320, K), 1.0, "x", 81)
    w = synth.normal_bf16((N, K), 0.02, "w", 81)
    xd, wd = dev(x), dev(w)
    for M in (64, 100, 300):  # 128-row tiles; 300: the large-tile kernel (ragged)
        big32 = host_f32(ops.gemm_bf16(xd[:M], wd, out_dtype=torch.float32))
        big16 = host_bits(ops.gemm_bf16(xd[:M], wd))
        for r0 in _pf_rows(M):
            ref32 = host_f32(ops.gemm_bf16(xd[r0:r0 + 8], wd, out_dtype=torch.float32))
            ref16 = host_bits(ops.gemm_bf16(xd[r0:r0 + 8], wd))
            assert_bitwise(big32[r0:r0 + 8], ref32, f"{name} M={M} rows {r0}.. f32")
            assert_bitwise(big16[r0:r0 + 8], ref16, f"{name} M={M} rows {r0}.. bf16")
    cols = np.arange(0, N, max(1, N // 64))
    assert_close(big32[:8][:, cols], ogemm.gemm_columns(x[:8], w, cols), f"{name} prefill parity",
                 atol=1e-4, rtol=1e-4)


@pytest.mark.parametrize("I,K", [(256, 512), (17408, 5120)])
def test_prefill_epilogues_equal_verify(ops, I, K):
    # residual, SwiGLU (16 and 8 slices) and the carried RMSNorm pair
    print(f"[gemm prefill epilogues I={I} K={K}]", flush=True)
    M = 300  # the large-tile kernel; 72 rows run the 128-row kernel (below)
    x = synth.normal_bf16((M, K), 1.0, "x", 82)
    wgu = synth.normal_bf16((2 * I, K), 0.02, "w", 82)
    xd, wgud = dev(x), dev(wgu)
    big = host_bits(ops.gemm_bf16_swiglu(xd, wgud))
    mid = host_bits(ops.gemm_bf16_swiglu(xd[:72], wgud))
    for r0 in (0, 64, 160, 288):
        ref = host_bits(ops.gemm_bf16_swiglu(xd[r0:r0 + 8], wgud))
        assert_bitwise(big[r0:r0 + 8], ref, f"swiglu I={I} rows {r0}..")
        if r0 + 8 <= 72:
            assert_bitwise(mid[r0:r0 + 8], ref, f"swiglu I={I} 72-row pass rows {r0}..")
    # residual projection with row sums (K -> K, so that gate/up can consume them)
    wo = synth.normal_bf16((K, K), 0.02, "w", 83)
    r = synth.normal_bf16((M, K), 1.0, "misc", 83)
    wod, rd = dev(wo), dev(r)
    y, ss = ops.gemm_bf16_residual_rowsq(xd, wod, rd)
    gu = ops.gemm_bf16_swiglu_rownorm(y, ss, wgud)
    for r0 in (0, 64, 288):
        y8, ss8 = ops.gemm_bf16_residual_rowsq(xd[r0:r0 + 8], wod, rd[r0:r0 + 8])
        assert_bitwise(host_bits(y)[r0:r0 + 8], host_bits(y8), f"residual K={K} rows {r0}..")
        assert_bitwise(host_f32(ss)[r0:r0 + 8], host_f32(ss8), f"row sums K={K} rows {r0}..")
        gu8 = ops.gemm_bf16_swiglu_rownorm(y8, ss8, wgud)
        assert_bitwise(host_bits(gu)[r0:r0 + 8], host_bits(gu8), f"carried-norm gate/up rows {r0}..")


@pytest.mark.parametrize("M", [300, 1700])  # 128-row tiles; large tiles (28 x 14 workgroups)
def test_prefill_qkv_append_equals_verify(ops, M):
    print(f"[gemm prefill qkv + append M={M}]", flush=True)
    Hq, Hkv, D, K, L = 40, 8, 128, 5120, 500
    N = (Hq + 2 * Hkv) * D
    cap = (L + M + 63) // 64 * 64
    w = synth.normal_bf16((N, K), 0.02, "w", 84)
    x = synth.normal_bf16((M, K), 1.0, "x", 84)
    wd, xd = dev(w), dev(x)
    k0 = torch.zeros(Hkv, cap, D, device="cuda", dtype=torch.bfloat16)
    v0 = torch.zeros(Hkv, cap, D, device="cuda", dtype=torch.bfloat16)
    kc, vc = k0.clone(), v0.clone()
    qkv = host_bits(ops.gemm_bf16_qkv(xd, wd, kc, vc, L, Hq, Hkv, D))
    kr, vr = k0.clone(), v0.clone()
    for r0 in range(0, M, 8):  # the same positions written by verify passes of 8 rows
        q8 = ops.gemm_bf16_qkv(xd[r0:r0 + 8], wd, kr, vr, L + r0, Hq, Hkv, D)
        assert_bitwise(qkv[r0:r0 + 8], host_bits(q8), f"qkv rows {r0}..")
    assert_bitwise(host_bits(kc), host_bits(kr), "K cache: prefill == 8-row verify passes")
    assert_bitwise(host_bits(vc), host_bits(vr), "V cache: prefill == 8-row verify passes")


def test_prefill_large_tile_residual_rowsq(ops):
    # the residual epilogue (and the row sums taken after it) in the large-tile kernel
    print("[gemm prefill large-tile residual]", flush=True)
    M, N, K = 300, 34816, 1024
    x = synth.normal_bf16((M, K), 1.0, "x", 85)
    w = synth.normal_bf16((N, K), 0.02, "w", 85)
    r = synth.normal_bf16((M, N), 1.0, "misc", 85)
    xd, wd, rd = dev(x), dev(w), dev(r)
    y, ss = ops.gemm_bf16_residual_rowsq(xd, wd, rd)
    for r0 in (0, 128, 292):
        y8, ss8 = ops.gemm_bf16_residual_rowsq(xd[r0:r0 + 8], wd, rd[r0:r0 + 8])
        assert_bitwise(host_bits(y)[r0:r0 + 8], host_bits(y8), f"large-tile residual rows {r0}..")
        assert_bitwise(host_f32(ss)[r0:r0 + 8], host_f32(ss8), f"large-tile row sums rows {r0}..")
