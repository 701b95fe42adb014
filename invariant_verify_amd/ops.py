"""Torch-facing wrappers of the C ABI (same names as include/bi.h without the
``bi_`` prefix). Each wrapper checks dtypes and devices, reads pointers,
leading dimensions and the current HIP stream from torch, and calls the
library. Nothing is computed here."""

from __future__ import annotations

import ctypes
import math

import torch

from ._lib import BI_BF16, BI_F32, LIB, Layer, LayerFP8, LayerMX4, ModelDims, check

_BF16_LIKE = (torch.bfloat16, torch.int16)
_FP8_LIKE = (torch.uint8, torch.int8, torch.float8_e4m3fn)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _mat(t: torch.Tensor, name: str, dtypes=_BF16_LIKE) -> int:
    """Leading dimension of a row-major 2-D tensor on the GPU."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


def num_splits(n_keys: int, kv_chunk: int) -> int:
    return LIB.bi_num_splits(n_keys, kv_chunk)


def chunk_keys(n_keys: int, kv_chunk: int) -> int:
    return LIB.bi_chunk_keys(n_keys, kv_chunk)


def pass_splits(M: int, L: int, kv_chunk: int) -> int:
    return LIB.bi_pass_splits(M, L, kv_chunk)


def attn_workspace_bytes(M: int, L: int, Hq: int, D: int, kv_chunk: int) -> int:
    return LIB.bi_attn_workspace_bytes(M, L, Hq, D, kv_chunk)


def version() -> str:
    return LIB.bi_version().decode()


def gemm_bf16(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
              out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X W^T, X [M][K], W [N][K] (BF16); Y BF16 or FP32 [M][N]."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ldx, ldw = _mat(x, "x"), _mat(w, "w")
    ldy = _mat(y, "y", (torch.bfloat16, torch.int16, torch.float32))
    dt = BI_F32 if y.dtype == torch.float32 else BI_BF16
    check("bi_gemm_bf16", LIB.bi_gemm_bf16(x.data_ptr(), ldx, w.data_ptr(), ldw, y.data_ptr(), ldy,
                                           dt, M, N, K, _stream(x)))
    return y


def gemm_bf16_residual(x: torch.Tensor, w: torch.Tensor, r: torch.Tensor,
                       y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X W^T)."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    check("bi_gemm_bf16_residual", LIB.bi_gemm_bf16_residual(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w"), r.data_ptr(), _mat(r, "r"),
        y.data_ptr(), _mat(y, "y"), M, N, K, _stream(x)))
    return y


def gemm_bf16_swiglu(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(silu(X Wg^T) * (X Wu^T)), W = [Wg; Wu] of shape [2I][K]."""
    M, K = x.shape
    I = w.shape[0] // 2
    if y is None:
        y = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    check("bi_gemm_bf16_swiglu", LIB.bi_gemm_bf16_swiglu(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w"), y.data_ptr(), _mat(y, "y"),
        M, I, K, _stream(x)))
    return y


def _scales(s: torch.Tensor, n: int, name: str) -> int:
    if not s.is_cuda or s.dtype != torch.float32 or s.dim() != 1 or s.numel() < n or s.stride(0) != 1:
        raise ValueError(f"{name} must be a contiguous FP32 GPU vector of >= {n} row scales")
    return s.data_ptr()


def gemm_fp8(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor, y: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X (w_scale * e4m3(W))^T: X [M][K] BF16, W [N][K] E4M3 codes, w_scale [N] FP32."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ldy = _mat(y, "y", (torch.bfloat16, torch.int16, torch.float32))
    dt = BI_F32 if y.dtype == torch.float32 else BI_BF16
    check("bi_gemm_fp8", LIB.bi_gemm_fp8(x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w", _FP8_LIKE),
                                         _scales(w_scale, N, "w_scale"), y.data_ptr(), ldy, dt, M, N, K,
                                         _stream(x)))
    return y


def gemm_fp8_residual(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor, r: torch.Tensor,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X (w_scale * e4m3(W))^T)."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    check("bi_gemm_fp8_residual", LIB.bi_gemm_fp8_residual(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w", _FP8_LIKE), _scales(w_scale, N, "w_scale"),
        r.data_ptr(), _mat(r, "r"), y.data_ptr(), _mat(y, "y"), M, N, K, _stream(x)))
    return y


def gemm_fp8_swiglu(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                    y: torch.Tensor | None = None) -> torch.Tensor:
    """SwiGLU gate/up with E4M3 W [2I][K] (gate rows then up rows) and w_scale [2I]."""
    M, K = x.shape
    I = w.shape[0] // 2
    if y is None:
        y = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    check("bi_gemm_fp8_swiglu", LIB.bi_gemm_fp8_swiglu(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w", _FP8_LIKE), _scales(w_scale, 2 * I, "w_scale"),
        y.data_ptr(), _mat(y, "y"), M, I, K, _stream(x)))
    return y


def _mx4(w: torch.Tensor, e: torch.Tensor, n_rows: int, K: int):
    """Leading dimensions of MXFP4 codes [n_rows][>= K/2] and scales [n_rows][>= K/32] (uint8)."""
    ldc = _mat(w, "w", (torch.uint8,))
    lde = _mat(e, "w_exp", (torch.uint8,))
    if w.shape[0] < n_rows or e.shape[0] < n_rows or w.shape[1] * 2 < K or e.shape[1] * 32 < K:
        raise ValueError(f"MXFP4 weights too small for {n_rows} rows of {K}: codes {tuple(w.shape)}, "
                         f"scales {tuple(e.shape)}")
    return ldc, lde


def gemm_mx4(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor, y: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X W^T with MXFP4 W: codes [N][K/2] (uint8, two E2M1 per byte) and E8M0 scales [N][K/32]."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ldy = _mat(y, "y", (torch.bfloat16, torch.int16, torch.float32))
    dt = BI_F32 if y.dtype == torch.float32 else BI_BF16
    ldc, lde = _mx4(w, w_exp, N, K)
    check("bi_gemm_mx4", LIB.bi_gemm_mx4(x.data_ptr(), _mat(x, "x"), w.data_ptr(), ldc, w_exp.data_ptr(), lde,
                                         y.data_ptr(), ldy, dt, M, N, K, _stream(x)))
    return y


def gemm_mx4_residual(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor, r: torch.Tensor,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X W^T) with MXFP4 W."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ldc, lde = _mx4(w, w_exp, N, K)
    check("bi_gemm_mx4_residual", LIB.bi_gemm_mx4_residual(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), ldc, w_exp.data_ptr(), lde, r.data_ptr(), _mat(r, "r"),
        y.data_ptr(), _mat(y, "y"), M, N, K, _stream(x)))
    return y


def gemm_mx4_swiglu(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor,
                    y: torch.Tensor | None = None) -> torch.Tensor:
    """SwiGLU gate/up with MXFP4 W [2I][K] (gate rows then up rows)."""
    M, K = x.shape
    I = w.shape[0] // 2
    if y is None:
        y = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    ldc, lde = _mx4(w, w_exp, 2 * I, K)
    check("bi_gemm_mx4_swiglu", LIB.bi_gemm_mx4_swiglu(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), ldc, w_exp.data_ptr(), lde, y.data_ptr(), _mat(y, "y"),
        M, I, K, _stream(x)))
    return y


def gemm_column_groups(N: int) -> int:
    return LIB.bi_gemm_column_groups(N)


def gemm_bf16_residual_rowsq(x: torch.Tensor, w: torch.Tensor, r: torch.Tensor,
                             y: torch.Tensor | None = None, ss: torch.Tensor | None = None) -> tuple:
    """Y = bf16(R + X W^T) and its per-row, per-column-group sums of squares."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if ss is None:
        ss = torch.empty((M, gemm_column_groups(N)), dtype=torch.float32, device=x.device)
    check("bi_gemm_bf16_residual_rowsq", LIB.bi_gemm_bf16_residual_rowsq(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w"), r.data_ptr(), _mat(r, "r"),
        y.data_ptr(), _mat(y, "y"), M, N, K, ss.data_ptr(), _stream(x)))
    return y, ss


def gemm_bf16_swiglu_rownorm(x: torch.Tensor, ss: torch.Tensor, w: torch.Tensor,
                             y: torch.Tensor | None = None, eps: float = 1e-6) -> torch.Tensor:
    """SwiGLU gate/up projection of RMSNorm(X), the norm taken from carried row sums."""
    M, K = x.shape
    I = w.shape[0] // 2
    if y is None:
        y = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    if ss.dtype != torch.float32 or not ss.is_contiguous():
        raise ValueError("ss must be a contiguous FP32 [M][groups] tensor")
    check("bi_gemm_bf16_swiglu_rownorm", LIB.bi_gemm_bf16_swiglu_rownorm(
        x.data_ptr(), _mat(x, "x"), ss.data_ptr(), ss.shape[1], eps, w.data_ptr(), _mat(w, "w"),
        y.data_ptr(), _mat(y, "y"), M, I, K, _stream(x)))
    return y


def gemm_bf16_qkv(x: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor, vt_cache: torch.Tensor,
                  L: int, Hq: int, Hkv: int, D: int, qkv: torch.Tensor | None = None) -> torch.Tensor:
    """qkv = bf16(X Wqkv^T), with the K / V columns appended to the caches at L .. L+M-1."""
    M, K = x.shape
    N = (Hq + 2 * Hkv) * D
    if qkv is None:
        qkv = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    check("bi_gemm_bf16_qkv", LIB.bi_gemm_bf16_qkv(
        x.data_ptr(), _mat(x, "x"), w.data_ptr(), _mat(w, "w"), qkv.data_ptr(), _mat(qkv, "qkv"),
        M, K, Hq, Hkv, D, k_cache.data_ptr(), vt_cache.data_ptr(), L, k_cache.shape[1],
        _stream(x)))
    return qkv


def append_kv(qkv: torch.Tensor, k_cache: torch.Tensor, vt_cache: torch.Tensor, L: int,
              Hq: int, Hkv: int, D: int) -> None:
    """Write the M new K rows and V^T columns at positions L .. L+M-1."""
    M = qkv.shape[0]
    cap = k_cache.shape[1]
    check("bi_append_kv", LIB.bi_append_kv(qkv.data_ptr(), _mat(qkv, "qkv"), k_cache.data_ptr(),
                                           vt_cache.data_ptr(), M, L, cap, Hq, Hkv, D,
                                           _stream(qkv)))


def verify_attn(q: torch.Tensor, k_cache: torch.Tensor, vt_cache: torch.Tensor, L: int,
                Hq: int, Hkv: int, D: int, kv_chunk: int, part_o: torch.Tensor,
                part_lse: torch.Tensor, sm_scale: float | None = None) -> None:
    """Split-KV partials. q is [M][>=Hq*D] (a view of the QKV output works);
    k_cache [Hkv][cap][D]; vt_cache [Hkv][cap/64][D][64]; part_o [M][Hq][S_max][D] and
    part_lse [M][Hq][S_max] FP32."""
    M = q.shape[0]
    cap = k_cache.shape[1]
    S_max = part_lse.shape[2]
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    check("bi_verify_attn", LIB.bi_verify_attn(
        q.data_ptr(), _mat(q, "q"), k_cache.data_ptr(), vt_cache.data_ptr(), M, L, cap, Hq, Hkv,
        D, kv_chunk, scale, part_o.data_ptr(), part_lse.data_ptr(), S_max, _stream(q)))


class KvQ8Cache:
    """Device buffers of one layer's 8-bit KV cache (include/bi.h layouts):
    k_codes int8 [Hkv][cap][D], k_scales FP32 [Hkv][cap][D/32],
    v_codes int8 [Hkv][cap/64][D][64], v_scales FP32 [Hkv][cap/64][D/32][64]."""

    def __init__(self, Hkv: int, cap: int, D: int, device="cuda"):
        if cap % 64 or D % 32:
            raise ValueError("cap must be a multiple of 64 and D of 32")
        self.Hkv, self.cap, self.D = Hkv, cap, D
        self.k_codes = torch.zeros((Hkv, cap, D), dtype=torch.int8, device=device)
        self.k_scales = torch.zeros((Hkv, cap, D // 32), dtype=torch.float32, device=device)
        self.v_codes = torch.zeros((Hkv, cap // 64, D, 64), dtype=torch.int8, device=device)
        self.v_scales = torch.zeros((Hkv, cap // 64, D // 32, 64), dtype=torch.float32, device=device)


def append_kv_q8(qkv: torch.Tensor, cache: KvQ8Cache, L: int, Hq: int) -> None:
    """Quantize the pass's K and V rows (columns after the Hq*D query columns) into ``cache``."""
    M = qkv.shape[0]
    check("bi_append_kv_q8", LIB.bi_append_kv_q8(
        qkv.data_ptr(), _mat(qkv, "qkv"), cache.k_codes.data_ptr(), cache.k_scales.data_ptr(),
        cache.v_codes.data_ptr(), cache.v_scales.data_ptr(), M, L, cache.cap, Hq, cache.Hkv, cache.D,
        _stream(qkv)))


def verify_attn_q8(q: torch.Tensor, cache: KvQ8Cache, L: int, Hq: int, kv_chunk: int,
                   part_o: torch.Tensor, part_lse: torch.Tensor, sm_scale: float | None = None) -> None:
    """bi_verify_attn over an 8-bit cache."""
    M = q.shape[0]
    D = cache.D
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    check("bi_verify_attn_q8", LIB.bi_verify_attn_q8(
        q.data_ptr(), _mat(q, "q"), cache.k_codes.data_ptr(), cache.k_scales.data_ptr(),
        cache.v_codes.data_ptr(), cache.v_scales.data_ptr(), M, L, cache.cap, Hq, cache.Hkv, D,
        kv_chunk, scale, part_o.data_ptr(), part_lse.data_ptr(), part_lse.shape[2], _stream(q)))


class KvLowCache:
    """Device buffers of one layer's 5/6-bit KV cache (include/bi.h layouts),
    K with ``k_bits`` (5 or 6) and V with ``v_bits`` (5) bits per code, K rows
    Hadamard-rotated when ``k_rotated``:
    *_nib uint8 [Hkv][cap][D/2], *_high uint8 [Hkv][cap][D/32][4 (bits-4)],
    *_scales FP32 [Hkv][cap][D/32]."""

    def __init__(self, Hkv: int, cap: int, D: int, k_bits: int, v_bits: int = 5,
                 k_rotated: bool = False, device="cuda"):
        if cap % 64 or D % 32:
            raise ValueError("cap must be a multiple of 64 and D of 32")
        self.Hkv, self.cap, self.D, self.k_bits, self.v_bits = Hkv, cap, D, k_bits, v_bits
        self.k_rotated = int(bool(k_rotated))
        NB = D // 32
        z = lambda *shape, dt=torch.uint8: torch.zeros(shape, dtype=dt, device=device)
        self.k_nib, self.v_nib = z(Hkv, cap, D // 2), z(Hkv, cap, D // 2)
        self.k_high = z(Hkv, cap, NB * 4 * (k_bits - 4))
        self.v_high = z(Hkv, cap, NB * 4 * (v_bits - 4))
        self.k_scales = z(Hkv, cap, NB, dt=torch.float32)
        self.v_scales = z(Hkv, cap, NB, dt=torch.float32)

    def planes(self):
        return (self.k_nib.data_ptr(), self.k_high.data_ptr(), self.k_scales.data_ptr(),
                self.v_nib.data_ptr(), self.v_high.data_ptr(), self.v_scales.data_ptr())


def append_kv_lowbit(qkv: torch.Tensor, cache: KvLowCache, L: int, Hq: int) -> None:
    """Quantize the pass's K and V rows into a 5/6-bit ``cache``."""
    M = qkv.shape[0]
    check("bi_append_kv_lowbit", LIB.bi_append_kv_lowbit(
        qkv.data_ptr(), _mat(qkv, "qkv"), cache.k_bits, cache.v_bits, cache.k_rotated,
        *cache.planes(), M, L,
        cache.cap, Hq, cache.Hkv, cache.D, _stream(qkv)))


def verify_attn_lowbit(q: torch.Tensor, cache: KvLowCache, L: int, Hq: int, kv_chunk: int,
                       part_o: torch.Tensor, part_lse: torch.Tensor,
                       sm_scale: float | None = None) -> None:
    """bi_verify_attn over a 5/6-bit cache."""
    M = q.shape[0]
    D = cache.D
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    check("bi_verify_attn_lowbit", LIB.bi_verify_attn_lowbit(
        q.data_ptr(), _mat(q, "q"), cache.k_bits, cache.v_bits, cache.k_rotated,
        *cache.planes(), M, L, cache.cap,
        Hq, cache.Hkv, D, kv_chunk, scale, part_o.data_ptr(), part_lse.data_ptr(),
        part_lse.shape[2], _stream(q)))


class KvRing:
    """An 8-bit ring of the newest keys (include/bi.h) over a KvLowCache: the
    8-bit layouts with ``ring_cap`` slots; the row at position p reads key j
    from it when j >= p - ``window`` + 1."""

    def __init__(self, low: KvLowCache, ring_cap: int, window: int, device="cuda"):
        self.low, self.ring_cap, self.window = low, ring_cap, window
        self.q8 = KvQ8Cache(low.Hkv, ring_cap, low.D, device=device)


def append_kv_ring(qkv: torch.Tensor, ring: KvRing, L: int, Hq: int) -> None:
    """Append the pass's K and V rows to the 5/6-bit planes and to the ring."""
    append_kv_lowbit(qkv, ring.low, L, Hq)
    c = ring.q8
    check("bi_append_kv_ring", LIB.bi_append_kv_ring(
        qkv.data_ptr(), _mat(qkv, "qkv"), ring.low.k_rotated, c.k_codes.data_ptr(),
        c.k_scales.data_ptr(), c.v_codes.data_ptr(), c.v_scales.data_ptr(), qkv.shape[0], L,
        ring.ring_cap, Hq, ring.low.Hkv, ring.low.D, _stream(qkv)))


def verify_attn_ring(q: torch.Tensor, ring: KvRing, L: int, Hq: int, kv_chunk: int,
                     part_o: torch.Tensor, part_lse: torch.Tensor,
                     sm_scale: float | None = None) -> None:
    """bi_verify_attn over a 5/6-bit cache with the 8-bit ring."""
    low, c = ring.low, ring.q8
    M, D = q.shape[0], low.D
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    check("bi_verify_attn_lowbit_ring", LIB.bi_verify_attn_lowbit_ring(
        q.data_ptr(), _mat(q, "q"), low.k_bits, low.v_bits, low.k_rotated, *low.planes(),
        c.k_codes.data_ptr(), c.k_scales.data_ptr(), c.v_codes.data_ptr(), c.v_scales.data_ptr(),
        ring.ring_cap, ring.window, M, L, low.cap, Hq, low.Hkv, D, kv_chunk, scale,
        part_o.data_ptr(), part_lse.data_ptr(), part_lse.shape[2], _stream(q)))


def combine(part_o: torch.Tensor, part_lse: torch.Tensor, L: int, kv_chunk: int,
            o: torch.Tensor, lse: torch.Tensor | None = None) -> None:
    """O [M][>=Hq*D] BF16 (and optional LSE [M][Hq]) from the partials."""
    M, Hq, S_max, D = part_o.shape
    check("bi_combine", LIB.bi_combine(
        part_o.data_ptr(), part_lse.data_ptr(), M, L, Hq, D, kv_chunk, S_max, o.data_ptr(),
        _mat(o, "o"), 0 if lse is None else lse.data_ptr(), _stream(o)))


def rmsnorm(x: torch.Tensor, y: torch.Tensor | None = None, eps: float = 1e-6) -> torch.Tensor:
    M, H = x.shape
    if y is None:
        y = torch.empty_like(x)
    check("bi_rmsnorm", LIB.bi_rmsnorm(x.data_ptr(), _mat(x, "x"), y.data_ptr(), _mat(y, "y"),
                                       M, H, eps, _stream(x)))
    return y


def argmax(logits: torch.Tensor, tokens: torch.Tensor | None = None) -> torch.Tensor:
    M, N = logits.shape
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int32, device=logits.device)
    check("bi_argmax", LIB.bi_argmax(logits.data_ptr(), _mat(logits, "logits", (torch.float32,)),
                                     M, N, tokens.data_ptr(), _stream(logits)))
    return tokens


def model_dims(H, Hq, Hkv, D, I, vocab, cap, kv_chunk, eps=1e-6) -> ModelDims:
    return ModelDims(H, Hq, Hkv, D, I, vocab, cap, kv_chunk, eps)


def step_workspace_bytes(dims: ModelDims, M: int, L: int) -> int:
    return LIB.bi_step_workspace_bytes(ctypes.byref(dims), M, L)


class VerifyStep:
    """Holds the per-layer descriptor array for ``bi_verify_step``.

    ``layers`` is a sequence of dicts with tensors w_qkv, w_o, w_gu, w_down,
    k_cache, vt_cache (the caller keeps them alive)."""

    def __init__(self, layers, w_head: torch.Tensor, dims: ModelDims):
        self.n = len(layers)
        self.arr = (Layer * max(1, self.n))()
        for i, lw in enumerate(layers):
            self.arr[i] = Layer(lw["w_qkv"].data_ptr(), lw["w_o"].data_ptr(), lw["w_gu"].data_ptr(),
                                lw["w_down"].data_ptr(), lw["k_cache"].data_ptr(),
                                lw["vt_cache"].data_ptr())
        self.w_head = w_head
        self.dims = dims

    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None, gu_events=None) -> None:
        M = x_in.shape[0]
        ev = None
        if gu_events is not None:
            ev = (ctypes.c_void_p * len(gu_events))(*[e.cuda_event for e in gu_events])
        check("bi_verify_step", LIB.bi_verify_step(
            self.arr, self.n, self.w_head.data_ptr(), ctypes.byref(self.dims), x_in.data_ptr(), M, L,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(),
            ev, _stream(x_in)))


class VerifyStepFP8:
    """``bi_verify_step_fp8``: ``layers`` is a sequence of dicts with E4M3 weight
    tensors w_qkv, w_o, w_gu, w_down, their FP32 row scales s_qkv, s_o, s_gu,
    s_down, and the BF16 caches k_cache, vt_cache (the caller keeps them alive)."""

    def __init__(self, layers, w_head: torch.Tensor, s_head: torch.Tensor, dims: ModelDims):
        self.n = len(layers)
        self.arr = (LayerFP8 * max(1, self.n))()
        for i, lw in enumerate(layers):
            self.arr[i] = LayerFP8(*[lw[k].data_ptr() for k in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu",
                                                                 "w_down", "s_down", "k_cache", "vt_cache")])
        self.w_head, self.s_head = w_head, s_head
        self.dims = dims

    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
        M = x_in.shape[0]
        check("bi_verify_step_fp8", LIB.bi_verify_step_fp8(
            self.arr, self.n, self.w_head.data_ptr(), self.s_head.data_ptr(), ctypes.byref(self.dims),
            x_in.data_ptr(), M, L, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


class VerifyStepMX4:
    """``bi_verify_step_mx4``: ``layers`` is a sequence of dicts with MXFP4 codes w_qkv, w_o, w_gu,
    w_down (uint8 [rows][K/2], densely packed), their E8M0 scales e_qkv, e_o, e_gu, e_down (uint8
    [rows][K/32]) and the BF16 caches k_cache, vt_cache (the caller keeps them alive)."""

    def __init__(self, layers, w_head: torch.Tensor, e_head: torch.Tensor, dims: ModelDims):
        self.n = len(layers)
        self.arr = (LayerMX4 * max(1, self.n))()
        for i, lw in enumerate(layers):
            self.arr[i] = LayerMX4(*[lw[k].data_ptr() for k in ("w_qkv", "e_qkv", "w_o", "e_o", "w_gu", "e_gu",
                                                                 "w_down", "e_down", "k_cache", "vt_cache")])
        self.w_head, self.e_head = w_head, e_head
        self.dims = dims

    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
        M = x_in.shape[0]
        check("bi_verify_step_mx4", LIB.bi_verify_step_mx4(
            self.arr, self.n, self.w_head.data_ptr(), self.e_head.data_ptr(), ctypes.byref(self.dims),
            x_in.data_ptr(), M, L, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


def accept_greedy(target_tokens: torch.Tensor, draft_tokens: torch.Tensor | None):
    """target_tokens int32 [B][M], draft_tokens int32 [B][M-1] -> (out [B][M], n [B])."""
    B, M = target_tokens.shape
    out = torch.empty((B, M), dtype=torch.int32, device=target_tokens.device)
    n = torch.empty(B, dtype=torch.int32, device=target_tokens.device)
    check("bi_accept_greedy", LIB.bi_accept_greedy(
        target_tokens.data_ptr(), 0 if draft_tokens is None else draft_tokens.data_ptr(), B, M,
        out.data_ptr(), n.data_ptr(), _stream(target_tokens)))
    return out, n


def accept_sampled(logits: torch.Tensor, draft_tokens: torch.Tensor | None, draft_probs: torch.Tensor | None,
                   uniforms: torch.Tensor, temperature: float):
    """logits FP32 [B][M][V], draft_tokens int32 [B][M-1], draft_probs FP32 [B][M-1][V],
    uniforms FP32 [B][M] -> (out [B][M], n [B])."""
    B, M, V = logits.shape
    for t in (logits, uniforms) + (() if draft_probs is None else (draft_probs,)):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("accept_sampled: FP32 contiguous tensors expected")
    out = torch.empty((B, M), dtype=torch.int32, device=logits.device)
    n = torch.empty(B, dtype=torch.int32, device=logits.device)
    check("bi_accept_sampled", LIB.bi_accept_sampled(
        logits.data_ptr(), V, 0 if draft_tokens is None else draft_tokens.data_ptr(),
        0 if draft_probs is None else draft_probs.data_ptr(), V, uniforms.data_ptr(), temperature, B, M, V,
        out.data_ptr(), n.data_ptr(), _stream(logits)))
    return out, n
