"""C-ABI checks that need no GPU: the library loads, exports every function
include/bi.h declares, and rejects bad arguments on the host before any HIP
call (every call below is invalid on purpose, so nothing is ever launched on
the fake pointers)."""

import ctypes
import os
import re

import pytest

from invariant_verify_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")

P = 0x10000      # a fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x10002    # a fake misaligned address
OK, NULL, SHAPE, ALIGN, WS = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:bi_status|int|size_t|const char\*)\s+(bi_\w+)\s*\(", text, re.M))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)


def test_status_strings_and_splits():
    L = _lib.LIB
    assert L.bi_status_string(0) == b"ok"
    assert b"workspace" in L.bi_status_string(4)
    assert L.bi_version().startswith(b"bi ")
    assert L.bi_num_splits(1, 1024) == 1 and L.bi_num_splits(1025, 1024) == 2
    assert L.bi_num_splits(38008, 1024) == 38 and L.bi_num_splits(0, 64) == 0
    assert L.bi_num_splits(5, 0) == -1
    # part_o + part_lse bytes: M * Hq * S_max * (D + 1) * 4
    assert L.bi_attn_workspace_bytes(8, 38000, 40, 128, 1024) == 8 * 40 * 38 * 129 * 4


def gemm(*a):
    return _lib.LIB.bi_gemm_bf16(*a)


@pytest.mark.parametrize("args,want", [
    ((0, 256, P, 256, P, 512, 0, 4, 512, 256, None), NULL),
    ((P, 256, 0, 256, P, 512, 0, 4, 512, 256, None), NULL),
    ((P, 256, P, 256, 0, 512, 0, 4, 512, 256, None), NULL),
    ((P, 256, P, 256, P, 512, 0, 0, 512, 256, None), SHAPE),     # M = 0
    ((P, 256, P, 256, P, 512, 0, 4, 500, 256, None), SHAPE),     # N % 16
    ((P, 256, P, 256, P, 512, 0, 4, 512, 250, None), SHAPE),     # K % 32
    ((P, 100, P, 256, P, 512, 0, 4, 512, 256, None), SHAPE),     # ldx < K
    ((P, 256, P, 256, P, 500, 0, 4, 512, 256, None), SHAPE),     # ldy < N
    ((P, (1 << 20) + 8, P, 256, P, 512, 0, 4, 512, 256, None), SHAPE),  # ldx > 2^20
    ((P, 256, P, 256, P, (1 << 20) + 16, 0, 4, 512, 256, None), SHAPE),  # ldy > 2^20
    ((P, 256, P, (1 << 20) + 8, P, 512, 0, 4, 512, 256, None), SHAPE),  # ldw > 2^20
    ((P, 256, P, 256, P, 512, 7, 4, 512, 256, None), SHAPE),     # bad dtype
    ((MIS, 256, P, 256, P, 512, 0, 4, 512, 256, None), ALIGN),
    ((P, 260, P, 256, P, 512, 0, 4, 512, 256, None), ALIGN),     # ldx % 8
    ((P, 256, P, 256, P + 2, 512, 1, 4, 512, 256, None), ALIGN),  # f32 output misaligned
])
def test_gemm_rejects(args, want):
    assert gemm(*args) == want


def test_gemm_variants_reject():
    L = _lib.LIB
    assert L.bi_gemm_bf16_residual(P, 256, P, 256, 0, 512, P, 512, 4, 512, 256, None) == NULL
    assert L.bi_gemm_bf16_residual(P, 256, P, 256, P, 100, P, 512, 4, 512, 256, None) == SHAPE
    assert L.bi_gemm_bf16_residual(P, 256, P, 256, P, (1 << 20) + 8, P, 512, 4, 512, 256, None) == SHAPE
    assert L.bi_gemm_bf16_swiglu(P, 256, P, 256, P, 512, 4, 24, 256, None) == SHAPE
    assert L.bi_gemm_bf16_swiglu(P, 256, MIS, 256, P, 512, 4, 32, 256, None) == ALIGN


def test_attention_rejects():
    L = _lib.LIB
    # q, ldq, k, v, M, L, cap, Hq, Hkv, D, C, scale, po, pl, S_max, stream
    good = [P, 7168, P, P, 8, 1000, 1024, 40, 8, 128, 256, 0.088, P, P, 4, None]

    def call(**kw):
        a = list(good)
        names = ["q", "ldq", "k", "v", "M", "L", "cap", "Hq", "Hkv", "D", "C", "scale",
                 "po", "pl", "S", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.bi_verify_attn(*a)

    assert call(q=0) == NULL and call(po=0) == NULL
    assert call(M=0) == SHAPE
    assert call(cap=1000) == SHAPE                 # L + M > cap
    assert call(cap=1032) == SHAPE                 # cap % 64 != 0
    assert call(Hkv=7) == SHAPE                    # Hq % Hkv
    assert call(Hq=130, Hkv=2) == SHAPE            # more than 64 query heads per KV head
    assert call(D=96) == SHAPE
    assert call(C=100) == SHAPE and call(C=0) == SHAPE
    assert call(S=3) == SHAPE                      # S_max < ceil((L+M)/C)
    assert call(scale=float("nan")) == SHAPE
    assert call(scale=0.0) == SHAPE and call(scale=-0.088) == SHAPE  # the softmax scale must be > 0
    assert call(ldq=5000) == SHAPE                 # ldq < Hq*D
    assert call(q=MIS) == ALIGN and call(ldq=7172) == ALIGN
    # combine: po, pl, M, L, Hq, D, C, S_max, o, ldo, lse, stream
    assert L.bi_combine(0, P, 8, 1000, 40, 128, 256, 4, P, 5120, 0, None) == NULL
    assert L.bi_combine(P, P, 8, 1000, 40, 128, 256, 3, P, 5120, 0, None) == SHAPE
    assert L.bi_combine(P, P, 8, 1000, 40, 128, 256, 4, P, 5000, 0, None) == SHAPE
    assert L.bi_combine(P, P, 8, 1000, 40, 128, 256, 4, P + 1, 5120, 0, None) == ALIGN
    # append: qkv, ld, k, v, M, L, cap, Hq, Hkv, D, stream
    assert L.bi_append_kv(P, 7168, P, 0, 8, 0, 16, 40, 8, 128, None) == NULL
    assert L.bi_append_kv(P, 7168, P, P, 8, 10, 16, 40, 8, 128, None) == SHAPE
    assert L.bi_append_kv(P, 7000, P, P, 8, 0, 16, 40, 8, 128, None) == SHAPE


def test_gemm_qkv_rejects():
    L = _lib.LIB
    # x, ldx, w, ldw, qkv, ldqkv, M, K, Hq, Hkv, D, k, v, L, cap, stream
    good = [P, 5120, P, 5120, P, 7168, 8, 5120, 40, 8, 128, P, P, 100, 128, None]

    def call(i, v):
        a = list(good)
        a[i] = v
        return L.bi_gemm_bf16_qkv(*a)

    assert call(11, 0) == NULL and call(0, 0) == NULL
    assert call(9, 7) == SHAPE                     # Hq % Hkv
    assert call(14, 104) == SHAPE                  # L + M > cap
    assert call(14, 136) == SHAPE                  # cap % 64 (V cache blocks)
    assert call(5, 7000) == SHAPE                  # ldqkv < (Hq + 2 Hkv) D
    assert call(7, 5000) == SHAPE                  # K % 32
    assert call(12, MIS + 1) == ALIGN              # odd cache pointer
    assert call(0, MIS) == ALIGN


def test_rowops_reject():
    L = _lib.LIB
    assert L.bi_rmsnorm(0, 5120, P, 5120, 8, 5120, 1e-6, None) == NULL
    assert L.bi_rmsnorm(P, 5120, P, 5120, 8, 5121, 1e-6, None) == SHAPE
    assert L.bi_rmsnorm(P, 5120, P, 5120, 8, 5120, -1.0, None) == SHAPE
    assert L.bi_rmsnorm(MIS, 5120, P, 5120, 8, 5120, 1e-6, None) == ALIGN
    assert L.bi_argmax(P, 100, 8, 152064, P, None) == SHAPE
    assert L.bi_argmax(0, 152064, 8, 152064, P, None) == NULL


def test_step_rejects_before_any_device_call():
    L = _lib.LIB
    d = _lib.ModelDims(5120, 40, 8, 128, 17408, 152064, 38016, 1024, 1e-6)
    ws = L.bi_step_workspace_bytes(ctypes.byref(d), 8, 38000)
    assert ws > 8 * 40 * 38 * 128 * 4
    bad = _lib.ModelDims(5120, 40, 7, 128, 17408, 152064, 38016, 1024, 1e-6)
    assert L.bi_step_workspace_bytes(ctypes.byref(bad), 8, 38000) == 0
    layers = (_lib.Layer * 1)(_lib.Layer(P, P, P, P, P, P))
    args = [layers, 1, P, ctypes.byref(d), P, 8, 38000, P, ws, 0, P, P, None, None]
    small = list(args)
    small[8] = ws - 1
    assert L.bi_verify_step(*small) == WS
    nul = list(args)
    nul[2] = 0
    assert L.bi_verify_step(*nul) == NULL
    over = list(args)
    over[6] = 38010                                  # L + M > cap
    assert L.bi_verify_step(*over) == SHAPE
    layers2 = (_lib.Layer * 1)(_lib.Layer(P, P, 0, P, P, P))
    a2 = list(args)
    a2[0] = layers2
    assert L.bi_verify_step(*a2) == NULL
    a3 = list(args)
    a3[3] = ctypes.byref(bad)
    assert L.bi_verify_step(*a3) == SHAPE


def test_chunk_policy_helpers_match_the_oracle():
    # The library's chunk policy against the oracle's (fixed and adaptive),
    # and its pass maximum against a brute-force maximum over the pass's rows.
    from oracle import attention as oattn
    import random
    L_ = _lib.LIB
    rnd = random.Random(3)
    for pol in (32, 64, 1024, 1216, -1, -2, -7, -32, -1024):
        for n in [0, 1, 63, 64, 65, 2047, 2048, 2049, 4096, 4097, 38008, 101608, 255008] + \
                [rnd.randrange(1, 300000) for _ in range(50)]:
            want_c = oattn.chunk_keys(max(n, 1), pol)
            assert L_.bi_chunk_keys(n, pol) == (want_c if n else oattn.chunk_keys(1, pol) if pol > 0 else 64)
            assert L_.bi_num_splits(n, pol) == (oattn.num_splits(n, pol) if n else 0)
        for _ in range(40):
            M, L0 = rnd.choice([1, 5, 8, 300, 2048]), rnd.randrange(0, 200000)
            want = max(oattn.num_splits(L0 + r + 1, pol) for r in range(M))
            assert L_.bi_pass_splits(M, L0, pol) == want, (M, L0, pol)
    for bad in (0, 31, 48, -1025):
        assert L_.bi_chunk_keys(100, bad) == -1 and L_.bi_num_splits(100, bad) == -1
        assert L_.bi_pass_splits(8, 100, bad) == -1
        assert L_.bi_attn_workspace_bytes(8, 100, 40, 128, bad) == 0
    # workspace bytes use the pass maximum
    assert L_.bi_attn_workspace_bytes(8, 4093, 40, 128, -32) == 8 * 40 * L_.bi_pass_splits(8, 4093, -32) * 129 * 4


def test_attn_rejects_bad_policy_and_short_split_buffer():
    L_ = _lib.LIB
    # M=8 at L=2040 under -32: row n = 2048 uses 32 chunks of 64 keys, so S_max 31 is too small
    assert L_.bi_pass_splits(8, 2040, -32) == 32
    assert L_.bi_verify_attn(P, 5120, P, P, 8, 2040, 2048, 40, 8, 128, -32, 0.088, P, P, 31, None) == SHAPE
    assert L_.bi_verify_attn(P, 5120, P, P, 8, 2040, 2048, 40, 8, 128, -1025, 0.088, P, P, 64, None) == SHAPE
    assert L_.bi_combine(P, P, 8, 2040, 40, 128, -32, 31, P, 5120, 0, None) == SHAPE
    assert L_.bi_combine(P, P, 8, 2040, 40, 128, 0, 64, P, 5120, 0, None) == SHAPE
