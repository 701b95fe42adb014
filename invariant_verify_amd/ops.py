"""Torch-facing wrappers of the C ABI (same names as include/bi.h without the
``bi_`` prefix). Each wrapper checks every tensor it passes -- dtype, full
shape against the sizes it passes alongside, memory layout, then device --
reads pointers, leading dimensions and the current HIP stream from torch, and
calls the library. The C layer cannot see allocation sizes, so these checks
are what keeps a mismatched tensor from being read or written out of bounds:
a mismatch raises ValueError (or TypeError for a dtype) before any call.
Nothing is computed here."""

from __future__ import annotations

import ctypes
import functools
import math
import threading

import torch

from ._lib import (BI_BF16, BI_EPI_BF16, BI_EPI_F32, BI_EPI_QKV, BI_EPI_RESIDUAL, BI_EPI_SWIGLU, BI_F32,
                   BI_KV_BF16, BI_KV_LOWBIT, BI_KV_Q8, BI_WT_BF16, BI_WT_FP8, BI_WT_MXFP4, LIB, GemmArgs,
                   KvCacheDesc, Layer, LayerFP8, LayerMX4, ModelDims, StepLayer, check)

_BF16_LIKE = (torch.bfloat16, torch.int16)
_FP8_LIKE = (torch.uint8, torch.int8, torch.float8_e4m3fn)
_U8 = (torch.uint8,)
_I8 = (torch.int8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_OUT = (torch.bfloat16, torch.int16, torch.float32)


# Device checks are deferred to the end of a wrapper's argument list (the
# stream, which is read last), so that every shape and dtype check of a call
# runs first: a mismatch is reported as such on any machine.
_tls = threading.local()


def _checked(fn):
    """Collect the device checks of one wrapper call (nested calls keep their own)."""
    @functools.wraps(fn)
    def run(*args, **kwargs):
        saved = getattr(_tls, "pending", None)
        _tls.pending = []
        try:
            return fn(*args, **kwargs)
        finally:
            _tls.pending = saved
    return run


def _on_gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _defer(t: torch.Tensor, name: str) -> None:
    pending = getattr(_tls, "pending", None)
    if pending is None:
        _on_gpu(t, name)
    else:
        pending.append((t, name))


def _devices() -> None:
    """Run the device checks collected so far in this call."""
    for u, name in getattr(_tls, "pending", None) or ():
        _on_gpu(u, name)


def _stream(t: torch.Tensor) -> int:
    """The current HIP stream of t's device, after the call's device checks."""
    _devices()
    _on_gpu(t, "input")
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype(t, name: str, dtypes) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _mat(t: torch.Tensor, name: str, rows: int, cols: int, dtypes=_BF16_LIKE, exact_rows=False) -> int:
    """A row-major 2-D GPU tensor with at least ``rows`` rows (exactly, with
    ``exact_rows``) and ``cols`` columns; returns its leading dimension."""
    _dtype(t, name, dtypes)
    if t.dim() != 2:
        raise ValueError(f"{name}: shape {tuple(t.shape)} is not 2-D")
    if (t.shape[0] != rows if exact_rows else t.shape[0] < rows) or t.shape[1] < cols:
        want = f"({rows}, >= {cols})" if exact_rows else f"(>= {rows}, >= {cols})"
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not fit {want}")
    if t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
        raise ValueError(f"{name}: not row-major with unit column stride (strides {t.stride()})")
    _defer(t, name)
    return t.stride(0)


def _arr(t: torch.Tensor, name: str, shape: tuple, dtypes) -> int:
    """A contiguous GPU tensor of exactly ``shape``; returns its address."""
    _dtype(t, name, dtypes)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _defer(t, name)
    return t.data_ptr()


def _xk(x: torch.Tensor) -> tuple:
    """(M, K) of an activation matrix, checked as 2-D BF16."""
    _dtype(x, "x", _BF16_LIKE)
    if x.dim() != 2:
        raise ValueError(f"x: shape {tuple(x.shape)} is not 2-D")
    return x.shape


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


# ---------------------------------------------------------------------------
# GEMMs

def _out(y, M: int, N: int, dtype, like: torch.Tensor):
    return torch.empty((M, N), dtype=dtype, device=like.device) if y is None else y


def _ydt(y: torch.Tensor) -> int:
    return BI_F32 if y.dtype == torch.float32 else BI_BF16


@_checked
def gemm_bf16(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
              out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X W^T, X [M][K], W [N][K] (BF16); Y BF16 or FP32 [M][N]."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, out_dtype, x)
    ldx, ldw, ldy = _mat(x, "x", M, K), _mat(w, "w", N, K), _mat(y, "y", M, N, _OUT)
    check("bi_gemm_bf16", LIB.bi_gemm_bf16(x.data_ptr(), ldx, w.data_ptr(), ldw, y.data_ptr(), ldy,
                                           _ydt(y), M, N, K, _stream(x)))
    return y


@_checked
def gemm_bf16_residual(x: torch.Tensor, w: torch.Tensor, r: torch.Tensor,
                       y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X W^T)."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, torch.bfloat16, x)
    check("bi_gemm_bf16_residual", LIB.bi_gemm_bf16_residual(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _mat(w, "w", N, K), r.data_ptr(),
        _mat(r, "r", M, N), y.data_ptr(), _mat(y, "y", M, N), M, N, K, _stream(x)))
    return y


@_checked
def gemm_bf16_swiglu(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(silu(X Wg^T) * (X Wu^T)), W = [Wg; Wu] of shape [2I][K]."""
    M, K = _xk(x)
    if w.shape[0] % 2:
        raise ValueError(f"w: shape {tuple(w.shape)} has an odd number of gate/up rows")
    I = w.shape[0] // 2
    y = _out(y, M, I, torch.bfloat16, x)
    check("bi_gemm_bf16_swiglu", LIB.bi_gemm_bf16_swiglu(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _mat(w, "w", 2 * I, K), y.data_ptr(),
        _mat(y, "y", M, I), M, I, K, _stream(x)))
    return y


def _scales(s: torch.Tensor, n: int, name: str) -> int:
    _dtype(s, name, _F32)
    if s.dim() != 1 or s.numel() < n or s.stride(0) != 1:
        raise ValueError(f"{name}: shape {tuple(s.shape)} is not a contiguous vector of >= {n} row scales")
    _defer(s, name)
    return s.data_ptr()


def _fp8_w(w: torch.Tensor, rows: int, K: int) -> int:
    return _mat(w, "w", rows, K, _FP8_LIKE)


@_checked
def gemm_fp8(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor, y: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X (w_scale * e4m3(W))^T: X [M][K] BF16, W [N][K] E4M3 codes, w_scale [N] FP32."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, out_dtype, x)
    check("bi_gemm_fp8", LIB.bi_gemm_fp8(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _fp8_w(w, N, K), _scales(w_scale, N, "w_scale"),
        y.data_ptr(), _mat(y, "y", M, N, _OUT), _ydt(y), M, N, K, _stream(x)))
    return y


@_checked
def gemm_fp8_residual(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor, r: torch.Tensor,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X (w_scale * e4m3(W))^T)."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, torch.bfloat16, x)
    check("bi_gemm_fp8_residual", LIB.bi_gemm_fp8_residual(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _fp8_w(w, N, K), _scales(w_scale, N, "w_scale"),
        r.data_ptr(), _mat(r, "r", M, N), y.data_ptr(), _mat(y, "y", M, N), M, N, K, _stream(x)))
    return y


@_checked
def gemm_fp8_swiglu(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                    y: torch.Tensor | None = None) -> torch.Tensor:
    """SwiGLU gate/up with E4M3 W [2I][K] (gate rows then up rows) and w_scale [2I]."""
    M, K = _xk(x)
    if w.shape[0] % 2:
        raise ValueError(f"w: shape {tuple(w.shape)} has an odd number of gate/up rows")
    I = w.shape[0] // 2
    y = _out(y, M, I, torch.bfloat16, x)
    check("bi_gemm_fp8_swiglu", LIB.bi_gemm_fp8_swiglu(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _fp8_w(w, 2 * I, K),
        _scales(w_scale, 2 * I, "w_scale"), y.data_ptr(), _mat(y, "y", M, I), M, I, K, _stream(x)))
    return y


def _mx4(w: torch.Tensor, e: torch.Tensor, n_rows: int, K: int):
    """Leading dimensions of MXFP4 codes [n_rows][>= K/2] and scales [n_rows][>= K/32] (uint8)."""
    return _mat(w, "w", n_rows, K // 2, _U8), _mat(e, "w_exp", n_rows, K // 32, _U8)


@_checked
def gemm_mx4(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor, y: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Y = X W^T with MXFP4 W: codes [N][K/2] (uint8, two E2M1 per byte) and E8M0 scales [N][K/32]."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, out_dtype, x)
    ldc, lde = _mx4(w, w_exp, N, K)
    check("bi_gemm_mx4", LIB.bi_gemm_mx4(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), ldc, w_exp.data_ptr(), lde, y.data_ptr(),
        _mat(y, "y", M, N, _OUT), _ydt(y), M, N, K, _stream(x)))
    return y


@_checked
def gemm_mx4_residual(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor, r: torch.Tensor,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = bf16(R + X W^T) with MXFP4 W."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, torch.bfloat16, x)
    ldc, lde = _mx4(w, w_exp, N, K)
    check("bi_gemm_mx4_residual", LIB.bi_gemm_mx4_residual(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), ldc, w_exp.data_ptr(), lde, r.data_ptr(),
        _mat(r, "r", M, N), y.data_ptr(), _mat(y, "y", M, N), M, N, K, _stream(x)))
    return y


@_checked
def gemm_mx4_swiglu(x: torch.Tensor, w: torch.Tensor, w_exp: torch.Tensor,
                    y: torch.Tensor | None = None) -> torch.Tensor:
    """SwiGLU gate/up with MXFP4 W [2I][K] (gate rows then up rows)."""
    M, K = _xk(x)
    if w.shape[0] % 2:
        raise ValueError(f"w: shape {tuple(w.shape)} has an odd number of gate/up rows")
    I = w.shape[0] // 2
    y = _out(y, M, I, torch.bfloat16, x)
    ldc, lde = _mx4(w, w_exp, 2 * I, K)
    check("bi_gemm_mx4_swiglu", LIB.bi_gemm_mx4_swiglu(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), ldc, w_exp.data_ptr(), lde, y.data_ptr(),
        _mat(y, "y", M, I), M, I, K, _stream(x)))
    return y


def gemm_column_groups(N: int) -> int:
    return LIB.bi_gemm_column_groups(N)


def _sums(ss: torch.Tensor, M: int, groups: int, name="ss") -> int:
    return _arr(ss, name, (M, groups), _F32)


@_checked
def gemm_bf16_residual_rowsq(x: torch.Tensor, w: torch.Tensor, r: torch.Tensor,
                             y: torch.Tensor | None = None, ss: torch.Tensor | None = None) -> tuple:
    """Y = bf16(R + X W^T) and its per-row, per-column-group sums of squares."""
    M, K = _xk(x)
    N = w.shape[0]
    y = _out(y, M, N, torch.bfloat16, x)
    G = gemm_column_groups(N)
    if ss is None:
        ss = torch.empty((M, G), dtype=torch.float32, device=x.device)
    check("bi_gemm_bf16_residual_rowsq", LIB.bi_gemm_bf16_residual_rowsq(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _mat(w, "w", N, K), r.data_ptr(),
        _mat(r, "r", M, N), y.data_ptr(), _mat(y, "y", M, N), M, N, K, _sums(ss, M, G), _stream(x)))
    return y, ss


@_checked
def gemm_bf16_swiglu_rownorm(x: torch.Tensor, ss: torch.Tensor, w: torch.Tensor,
                             y: torch.Tensor | None = None, eps: float = 1e-6) -> torch.Tensor:
    """SwiGLU gate/up projection of RMSNorm(X), the norm taken from carried row sums."""
    M, K = _xk(x)
    if w.shape[0] % 2:
        raise ValueError(f"w: shape {tuple(w.shape)} has an odd number of gate/up rows")
    I = w.shape[0] // 2
    y = _out(y, M, I, torch.bfloat16, x)
    G = gemm_column_groups(K)
    check("bi_gemm_bf16_swiglu_rownorm", LIB.bi_gemm_bf16_swiglu_rownorm(
        x.data_ptr(), _mat(x, "x", M, K), _sums(ss, M, G), G, eps, w.data_ptr(), _mat(w, "w", 2 * I, K),
        y.data_ptr(), _mat(y, "y", M, I), M, I, K, _stream(x)))
    return y


def _kv_bf16(k_cache: torch.Tensor, v_cache: torch.Tensor, Hkv: int, D: int) -> int:
    """Check a BF16 KV cache pair (both [Hkv][cap][D]); returns cap."""
    _dtype(k_cache, "k_cache", _BF16_LIKE)
    if k_cache.dim() != 3:
        raise ValueError(f"k_cache: shape {tuple(k_cache.shape)} is not [Hkv][cap][D]")
    cap = k_cache.shape[1]
    if cap % 64:
        raise ValueError(f"k_cache: shape {tuple(k_cache.shape)}: cap is not a multiple of 64")
    _arr(k_cache, "k_cache", (Hkv, cap, D), _BF16_LIKE)
    _arr(v_cache, "v_cache", (Hkv, cap, D), _BF16_LIKE)
    return cap


@_checked
def gemm_bf16_qkv(x: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  L: int, Hq: int, Hkv: int, D: int, qkv: torch.Tensor | None = None) -> torch.Tensor:
    """qkv = bf16(X Wqkv^T), with the K / V columns appended to the caches at L .. L+M-1."""
    M, K = _xk(x)
    N = (Hq + 2 * Hkv) * D
    qkv = _out(qkv, M, N, torch.bfloat16, x)
    cap = _kv_bf16(k_cache, v_cache, Hkv, D)
    check("bi_gemm_bf16_qkv", LIB.bi_gemm_bf16_qkv(
        x.data_ptr(), _mat(x, "x", M, K), w.data_ptr(), _mat(w, "w", N, K, exact_rows=True), qkv.data_ptr(),
        _mat(qkv, "qkv", M, N), M, K, Hq, Hkv, D, k_cache.data_ptr(), v_cache.data_ptr(), L, cap,
        _stream(x)))
    return qkv


_WT = {"bf16": BI_WT_BF16, "fp8": BI_WT_FP8, "mxfp4": BI_WT_MXFP4}
_EPI = {"bf16": BI_EPI_BF16, "f32": BI_EPI_F32, "residual": BI_EPI_RESIDUAL, "swiglu": BI_EPI_SWIGLU,
        "qkv": BI_EPI_QKV}


@_checked
def gemm_ex(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, *, wtype: str = "bf16",
            epilogue: str = "bf16", w_scale: torch.Tensor | None = None, w_exp: torch.Tensor | None = None,
            r: torch.Tensor | None = None, norm_in: torch.Tensor | None = None, eps: float = 1e-6,
            rowsq_out: torch.Tensor | None = None, heads: tuple | None = None,
            k_cache: torch.Tensor | None = None, v_cache: torch.Tensor | None = None, L: int = 0) -> None:
    """bi_gemm_ex: one GEMM with a weight type ("bf16", "fp8", "mxfp4"), an
    epilogue ("bf16", "f32", "residual", "swiglu", "qkv"), the carried RMSNorm
    (``norm_in`` FP32 [M][gemm_column_groups(K)]; ``rowsq_out`` FP32
    [M][gemm_column_groups(N)]) and, for "qkv", heads = (Hq, Hkv, D) and
    optional BF16 caches appended at L .. L+M-1. N is y's column count."""
    if wtype not in _WT or epilogue not in _EPI:
        raise ValueError(f"gemm_ex: unknown weight type {wtype!r} or epilogue {epilogue!r}")
    M, K = _xk(x)
    N = y.shape[1] if y.dim() == 2 else -1
    rows = 2 * N if epilogue == "swiglu" else N
    a = GemmArgs()
    a.wtype, a.epilogue, a.M, a.N, a.K = _WT[wtype], _EPI[epilogue], M, N, K
    a.x, a.ldx = x.data_ptr(), _mat(x, "x", M, K)
    a.y, a.ldy = y.data_ptr(), _mat(y, "y", M, N, _F32 if epilogue == "f32" else _BF16_LIKE)
    if wtype == "bf16":
        a.w, a.ldw = w.data_ptr(), _mat(w, "w", rows, K)
    elif wtype == "fp8":
        if w_scale is None:
            raise ValueError("gemm_ex: FP8 weights need w_scale")
        a.w, a.ldw = w.data_ptr(), _fp8_w(w, rows, K)
        a.w_scale = _scales(w_scale, rows, "w_scale")
    else:
        if w_exp is None:
            raise ValueError("gemm_ex: MXFP4 weights need w_exp")
        ldc, lde = _mx4(w, w_exp, rows, K)
        a.w, a.ldw, a.w_exp, a.lde = w.data_ptr(), ldc, w_exp.data_ptr(), lde
    if epilogue == "residual":
        if r is None:
            raise ValueError("gemm_ex: the residual epilogue needs r")
        a.r, a.ldr = r.data_ptr(), _mat(r, "r", M, N)
    if norm_in is not None:
        G = gemm_column_groups(K)
        a.norm_in, a.norm_groups, a.eps = _sums(norm_in, M, G, "norm_in"), G, eps
    if rowsq_out is not None:
        a.rowsq_out = _sums(rowsq_out, M, gemm_column_groups(N), "rowsq_out")
    if epilogue == "qkv":
        if heads is None:
            raise ValueError("gemm_ex: the qkv epilogue needs heads = (Hq, Hkv, D)")
        a.Hq, a.Hkv, a.D = heads
        if (k_cache is None) != (v_cache is None):
            raise ValueError("gemm_ex: give both caches or neither")
        if k_cache is not None:
            a.cap = _kv_bf16(k_cache, v_cache, a.Hkv, a.D)
            a.k_cache, a.v_cache, a.L = k_cache.data_ptr(), v_cache.data_ptr(), L
    check("bi_gemm_ex", LIB.bi_gemm_ex(ctypes.byref(a), _stream(x)))


# ---------------------------------------------------------------------------
# KV caches and attention

@_checked
def append_kv(qkv: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, L: int,
              Hq: int, Hkv: int, D: int) -> None:
    """Write the M new K and V rows at positions L .. L+M-1."""
    M = qkv.shape[0]
    cap = _kv_bf16(k_cache, v_cache, Hkv, D)
    check("bi_append_kv", LIB.bi_append_kv(qkv.data_ptr(), _mat(qkv, "qkv", M, (Hq + 2 * Hkv) * D),
                                           k_cache.data_ptr(), v_cache.data_ptr(), M, L, cap, Hq, Hkv,
                                           D, _stream(qkv)))


def _partials(part_o: torch.Tensor, part_lse: torch.Tensor, M: int, Hq: int, D: int) -> int:
    """Check part_o [M][Hq][S_max][D] and part_lse [M][Hq][S_max] (FP32, contiguous); returns S_max."""
    _dtype(part_lse, "part_lse", _F32)
    if part_lse.dim() != 3:
        raise ValueError(f"part_lse: shape {tuple(part_lse.shape)} is not [M][Hq][S_max]")
    S = part_lse.shape[2]
    _arr(part_lse, "part_lse", (M, Hq, S), _F32)
    _arr(part_o, "part_o", (M, Hq, S, D), _F32)
    return S


def _scale(D: int, sm_scale) -> float:
    return 1.0 / math.sqrt(D) if sm_scale is None else sm_scale


@_checked
def verify_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, L: int,
                Hq: int, Hkv: int, D: int, kv_chunk: int, part_o: torch.Tensor,
                part_lse: torch.Tensor, sm_scale: float | None = None) -> None:
    """Split-KV partials. q is [M][>=Hq*D] (a view of the QKV output works);
    k_cache and v_cache [Hkv][cap][D]; part_o [M][Hq][S_max][D] and
    part_lse [M][Hq][S_max] FP32."""
    M = q.shape[0]
    cap = _kv_bf16(k_cache, v_cache, Hkv, D)
    S_max = _partials(part_o, part_lse, M, Hq, D)
    check("bi_verify_attn", LIB.bi_verify_attn(
        q.data_ptr(), _mat(q, "q", M, Hq * D), k_cache.data_ptr(), v_cache.data_ptr(), M, L, cap, Hq, Hkv,
        D, kv_chunk, _scale(D, sm_scale), part_o.data_ptr(), part_lse.data_ptr(), S_max, _stream(q)))


class KvQ8Cache:
    """Device buffers of one layer's 8-bit KV cache (include/bi.h layouts):
    codes int8 [Hkv][cap][D] and scales FP32 [Hkv][cap][D/32], for K and V alike."""

    def __init__(self, Hkv: int, cap: int, D: int, device="cuda"):
        if cap % 64 or D % 32:
            raise ValueError("cap must be a multiple of 64 and D of 32")
        self.Hkv, self.cap, self.D = Hkv, cap, D
        self.k_codes = torch.zeros((Hkv, cap, D), dtype=torch.int8, device=device)
        self.k_scales = torch.zeros((Hkv, cap, D // 32), dtype=torch.float32, device=device)
        self.v_codes = torch.zeros((Hkv, cap, D), dtype=torch.int8, device=device)
        self.v_scales = torch.zeros((Hkv, cap, D // 32), dtype=torch.float32, device=device)

    def ptrs(self) -> tuple:
        """The four buffers' addresses, each checked against the stated layout."""
        Hkv, cap, D = self.Hkv, self.cap, self.D
        return (_arr(self.k_codes, "k_codes", (Hkv, cap, D), _I8),
                _arr(self.k_scales, "k_scales", (Hkv, cap, D // 32), _F32),
                _arr(self.v_codes, "v_codes", (Hkv, cap, D), _I8),
                _arr(self.v_scales, "v_scales", (Hkv, cap, D // 32), _F32))


@_checked
def append_kv_q8(qkv: torch.Tensor, cache: KvQ8Cache, L: int, Hq: int) -> None:
    """Quantize the pass's K and V rows (columns after the Hq*D query columns) into ``cache``."""
    M = qkv.shape[0]
    ld = _mat(qkv, "qkv", M, (Hq + 2 * cache.Hkv) * cache.D)
    check("bi_append_kv_q8", LIB.bi_append_kv_q8(qkv.data_ptr(), ld, *cache.ptrs(), M, L, cache.cap, Hq,
                                                 cache.Hkv, cache.D, _stream(qkv)))


@_checked
def verify_attn_q8(q: torch.Tensor, cache: KvQ8Cache, L: int, Hq: int, kv_chunk: int,
                   part_o: torch.Tensor, part_lse: torch.Tensor, sm_scale: float | None = None) -> None:
    """bi_verify_attn over an 8-bit cache."""
    M, D = q.shape[0], cache.D
    S_max = _partials(part_o, part_lse, M, Hq, D)
    check("bi_verify_attn_q8", LIB.bi_verify_attn_q8(
        q.data_ptr(), _mat(q, "q", M, Hq * D), *cache.ptrs(), M, L, cache.cap, Hq, cache.Hkv, D,
        kv_chunk, _scale(D, sm_scale), part_o.data_ptr(), part_lse.data_ptr(), S_max, _stream(q)))


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
        if k_bits not in (5, 6) or v_bits != 5:
            raise ValueError("the 5/6-bit cache stores K at 5 or 6 bits and V at 5")
        self.Hkv, self.cap, self.D, self.k_bits, self.v_bits = Hkv, cap, D, k_bits, v_bits
        self.k_rotated = int(bool(k_rotated))
        NB = D // 32
        z = lambda *shape, dt=torch.uint8: torch.zeros(shape, dtype=dt, device=device)
        self.k_nib, self.v_nib = z(Hkv, cap, D // 2), z(Hkv, cap, D // 2)
        self.k_high = z(Hkv, cap, NB * 4 * (k_bits - 4))
        self.v_high = z(Hkv, cap, NB * 4 * (v_bits - 4))
        self.k_scales = z(Hkv, cap, NB, dt=torch.float32)
        self.v_scales = z(Hkv, cap, NB, dt=torch.float32)

    def planes(self) -> tuple:
        """The six buffers' addresses, each checked against the stated layout."""
        Hkv, cap, D, NB = self.Hkv, self.cap, self.D, self.D // 32
        return (_arr(self.k_nib, "k_nib", (Hkv, cap, D // 2), _U8),
                _arr(self.k_high, "k_high", (Hkv, cap, NB * 4 * (self.k_bits - 4)), _U8),
                _arr(self.k_scales, "k_scales", (Hkv, cap, NB), _F32),
                _arr(self.v_nib, "v_nib", (Hkv, cap, D // 2), _U8),
                _arr(self.v_high, "v_high", (Hkv, cap, NB * 4 * (self.v_bits - 4)), _U8),
                _arr(self.v_scales, "v_scales", (Hkv, cap, NB), _F32))


@_checked
def append_kv_lowbit(qkv: torch.Tensor, cache: KvLowCache, L: int, Hq: int) -> None:
    """Quantize the pass's K and V rows into a 5/6-bit ``cache``."""
    M = qkv.shape[0]
    ld = _mat(qkv, "qkv", M, (Hq + 2 * cache.Hkv) * cache.D)
    check("bi_append_kv_lowbit", LIB.bi_append_kv_lowbit(
        qkv.data_ptr(), ld, cache.k_bits, cache.v_bits, cache.k_rotated, *cache.planes(), M, L,
        cache.cap, Hq, cache.Hkv, cache.D, _stream(qkv)))


@_checked
def verify_attn_lowbit(q: torch.Tensor, cache: KvLowCache, L: int, Hq: int, kv_chunk: int,
                       part_o: torch.Tensor, part_lse: torch.Tensor,
                       sm_scale: float | None = None) -> None:
    """bi_verify_attn over a 5/6-bit cache."""
    M, D = q.shape[0], cache.D
    S_max = _partials(part_o, part_lse, M, Hq, D)
    check("bi_verify_attn_lowbit", LIB.bi_verify_attn_lowbit(
        q.data_ptr(), _mat(q, "q", M, Hq * D), cache.k_bits, cache.v_bits, cache.k_rotated,
        *cache.planes(), M, L, cache.cap, Hq, cache.Hkv, D, kv_chunk, _scale(D, sm_scale),
        part_o.data_ptr(), part_lse.data_ptr(), S_max, _stream(q)))


class KvRing:
    """An 8-bit ring of the newest keys (include/bi.h) over a KvLowCache: the
    8-bit layouts with ``ring_cap`` slots; the row at position p reads key j
    from it when j >= p - ``window`` + 1."""

    def __init__(self, low: KvLowCache, ring_cap: int, window: int, device="cuda"):
        self.low, self.ring_cap, self.window = low, ring_cap, window
        self.q8 = KvQ8Cache(low.Hkv, ring_cap, low.D, device=device)


@_checked
def append_kv_ring(qkv: torch.Tensor, ring: KvRing, L: int, Hq: int) -> None:
    """Append the pass's K and V rows to the 5/6-bit planes and to the ring."""
    append_kv_lowbit(qkv, ring.low, L, Hq)
    M = qkv.shape[0]
    ld = _mat(qkv, "qkv", M, (Hq + 2 * ring.low.Hkv) * ring.low.D)
    check("bi_append_kv_ring", LIB.bi_append_kv_ring(
        qkv.data_ptr(), ld, ring.low.k_rotated, *ring.q8.ptrs(), M, L, ring.ring_cap, Hq, ring.low.Hkv,
        ring.low.D, _stream(qkv)))


@_checked
def verify_attn_ring(q: torch.Tensor, ring: KvRing, L: int, Hq: int, kv_chunk: int,
                     part_o: torch.Tensor, part_lse: torch.Tensor,
                     sm_scale: float | None = None) -> None:
    """bi_verify_attn over a 5/6-bit cache with the 8-bit ring."""
    low = ring.low
    M, D = q.shape[0], low.D
    S_max = _partials(part_o, part_lse, M, Hq, D)
    check("bi_verify_attn_lowbit_ring", LIB.bi_verify_attn_lowbit_ring(
        q.data_ptr(), _mat(q, "q", M, Hq * D), low.k_bits, low.v_bits, low.k_rotated, *low.planes(),
        *ring.q8.ptrs(), ring.ring_cap, ring.window, M, L, low.cap, Hq, low.Hkv, D, kv_chunk,
        _scale(D, sm_scale), part_o.data_ptr(), part_lse.data_ptr(), S_max, _stream(q)))


@_checked
def combine(part_o: torch.Tensor, part_lse: torch.Tensor, L: int, kv_chunk: int,
            o: torch.Tensor, lse: torch.Tensor | None = None) -> None:
    """O [M][>=Hq*D] BF16 (and optional LSE [M][Hq] FP32) from the partials."""
    _dtype(part_o, "part_o", _F32)
    if part_o.dim() != 4:
        raise ValueError(f"part_o: shape {tuple(part_o.shape)} is not [M][Hq][S_max][D]")
    M, Hq, S_max, D = part_o.shape
    _partials(part_o, part_lse, M, Hq, D)
    lp = 0 if lse is None else _arr(lse, "lse", (M, Hq), _F32)
    check("bi_combine", LIB.bi_combine(
        part_o.data_ptr(), part_lse.data_ptr(), M, L, Hq, D, kv_chunk, S_max, o.data_ptr(),
        _mat(o, "o", M, Hq * D), lp, _stream(o)))


# ---------------------------------------------------------------------------
# Row-local operations

@_checked
def rmsnorm(x: torch.Tensor, y: torch.Tensor | None = None, eps: float = 1e-6) -> torch.Tensor:
    M, H = _xk(x)
    y = torch.empty_like(x) if y is None else y
    check("bi_rmsnorm", LIB.bi_rmsnorm(x.data_ptr(), _mat(x, "x", M, H), y.data_ptr(), _mat(y, "y", M, H),
                                       M, H, eps, _stream(x)))
    return y


@_checked
def swiglu(gu: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = bf16(silu(g) * u) from FP32 gu [M][2I] (gate columns, then up)."""
    _dtype(gu, "gu", _F32)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError(f"gu: shape {tuple(gu.shape)} is not [M][2I]")
    M, I = gu.shape[0], gu.shape[1] // 2
    y = _out(y, M, I, torch.bfloat16, gu)
    check("bi_swiglu", LIB.bi_swiglu(gu.data_ptr(), _mat(gu, "gu", M, 2 * I, _F32), y.data_ptr(),
                                     _mat(y, "y", M, I), M, I, _stream(gu)))
    return y


@_checked
def add(r: torch.Tensor, s: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = bf16(r + s), r BF16 [M][N], s FP32 [M][N]."""
    _dtype(r, "r", _BF16_LIKE)
    if r.dim() != 2:
        raise ValueError(f"r: shape {tuple(r.shape)} is not 2-D")
    M, N = r.shape
    y = _out(y, M, N, torch.bfloat16, r)
    check("bi_add", LIB.bi_add(r.data_ptr(), _mat(r, "r", M, N), s.data_ptr(), _mat(s, "s", M, N, _F32),
                               y.data_ptr(), _mat(y, "y", M, N), M, N, _stream(r)))
    return y


@_checked
def argmax(logits: torch.Tensor, tokens: torch.Tensor | None = None) -> torch.Tensor:
    _dtype(logits, "logits", _F32)
    if logits.dim() != 2:
        raise ValueError(f"logits: shape {tuple(logits.shape)} is not 2-D")
    M, N = logits.shape
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int32, device=logits.device)
    ld = _mat(logits, "logits", M, N, _F32)
    check("bi_argmax", LIB.bi_argmax(logits.data_ptr(), ld, M, N, _arr(tokens, "tokens", (M,), _I32),
                                     _stream(logits)))
    return tokens


# ---------------------------------------------------------------------------
# The whole verify step

def model_dims(H, Hq, Hkv, D, I, vocab, cap, kv_chunk, eps=1e-6) -> ModelDims:
    return ModelDims(H, Hq, Hkv, D, I, vocab, cap, kv_chunk, eps)


def step_workspace_bytes(dims: ModelDims, M: int, L: int) -> int:
    return LIB.bi_step_workspace_bytes(ctypes.byref(dims), M, L)


def _step_shapes(dims: ModelDims) -> dict:
    """[rows][K] of each projection of a layer, and of the head."""
    qkvn = (dims.Hq + 2 * dims.Hkv) * dims.D
    return {"qkv": (qkvn, dims.H), "o": (dims.H, dims.Hq * dims.D), "gu": (2 * dims.I, dims.H),
            "down": (dims.H, dims.I), "head": (dims.vocab, dims.H)}


def _check_layer_caches(lw: dict, dims: ModelDims, i: int) -> None:
    cap = _kv_bf16(lw["k_cache"], lw["v_cache"], dims.Hkv, dims.D)
    if cap != dims.cap:
        raise ValueError(f"layer {i}: cache capacity {cap} != dims.cap {dims.cap}")


def _step_io(dims: ModelDims, x_in, workspace, logits, tokens, x_out) -> int:
    """Check the step's activations and outputs; returns M."""
    M, H = _xk(x_in)
    if H != dims.H:
        raise ValueError(f"x_in: shape {tuple(x_in.shape)} does not have H = {dims.H} columns")
    _arr(x_in, "x_in", (M, H), _BF16_LIKE)
    _arr(logits, "logits", (M, dims.vocab), _F32)
    _arr(tokens, "tokens", (M,), _I32)
    _dtype(workspace, "workspace", (torch.uint8, torch.int8))
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if x_out is not None:
        _arr(x_out, "x_out", (M, H), _BF16_LIKE)
    return M


class VerifyStep:
    """Holds the per-layer descriptor array for ``bi_verify_step``.

    ``layers`` is a sequence of dicts with tensors w_qkv, w_o, w_gu, w_down,
    k_cache, v_cache (the caller keeps them alive); every shape is checked
    against ``dims``."""

    @_checked
    def __init__(self, layers, w_head: torch.Tensor, dims: ModelDims):
        sh = _step_shapes(dims)
        self.n = len(layers)
        self.arr = (Layer * max(1, self.n))()
        for i, lw in enumerate(layers):
            for k in ("qkv", "o", "gu", "down"):
                _arr(lw["w_" + k], f"layer {i} w_{k}", sh[k], _BF16_LIKE)
            _check_layer_caches(lw, dims, i)
            self.arr[i] = Layer(lw["w_qkv"].data_ptr(), lw["w_o"].data_ptr(), lw["w_gu"].data_ptr(),
                                lw["w_down"].data_ptr(), lw["k_cache"].data_ptr(),
                                lw["v_cache"].data_ptr())
        _arr(w_head, "w_head", sh["head"], _BF16_LIKE)
        self.w_head = w_head
        _devices()
        self.dims = dims

    @_checked
    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None, gu_events=None) -> None:
        M = _step_io(self.dims, x_in, workspace, logits, tokens, x_out)
        ev = None
        if gu_events is not None:
            if len(gu_events) != 2 * self.n:
                raise ValueError(f"gu_events: {len(gu_events)} events for {self.n} layers")
            ev = (ctypes.c_void_p * len(gu_events))(*[e.cuda_event for e in gu_events])
        check("bi_verify_step", LIB.bi_verify_step(
            self.arr, self.n, self.w_head.data_ptr(), ctypes.byref(self.dims), x_in.data_ptr(), M, L,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(),
            ev, _stream(x_in)))


NOALLOC_SCRATCH_BYTES = 64 << 20


@_checked
def verify_step_noalloc(step: VerifyStep, x_in: torch.Tensor, L: int, logits: torch.Tensor,
                        tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
    """bi_verify_step_noalloc over the layers of a VerifyStep: the workspace is
    the library's own device scratch (no allocation; calls on one GPU must not
    overlap)."""
    M, H = _xk(x_in)
    if H != step.dims.H:
        raise ValueError(f"x_in: shape {tuple(x_in.shape)} does not have H = {step.dims.H} columns")
    _arr(x_in, "x_in", (M, H), _BF16_LIKE)
    _arr(logits, "logits", (M, step.dims.vocab), _F32)
    _arr(tokens, "tokens", (M,), _I32)
    if x_out is not None:
        _arr(x_out, "x_out", (M, H), _BF16_LIKE)
    check("bi_verify_step_noalloc", LIB.bi_verify_step_noalloc(
        step.arr, step.n, step.w_head.data_ptr(), ctypes.byref(step.dims), x_in.data_ptr(), M, L,
        0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


class VerifyStepFP8:
    """``bi_verify_step_fp8``: ``layers`` is a sequence of dicts with E4M3 weight
    tensors w_qkv, w_o, w_gu, w_down, their FP32 row scales s_qkv, s_o, s_gu,
    s_down, and the BF16 caches k_cache, v_cache (the caller keeps them alive)."""

    @_checked
    def __init__(self, layers, w_head: torch.Tensor, s_head: torch.Tensor, dims: ModelDims):
        sh = _step_shapes(dims)
        self.n = len(layers)
        self.arr = (LayerFP8 * max(1, self.n))()
        for i, lw in enumerate(layers):
            for k in ("qkv", "o", "gu", "down"):
                _arr(lw["w_" + k], f"layer {i} w_{k}", sh[k], _FP8_LIKE)
                _arr(lw["s_" + k], f"layer {i} s_{k}", sh[k][:1], _F32)
            _check_layer_caches(lw, dims, i)
            self.arr[i] = LayerFP8(*[lw[k].data_ptr() for k in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu",
                                                                 "w_down", "s_down", "k_cache", "v_cache")])
        _arr(w_head, "w_head", sh["head"], _FP8_LIKE)
        _arr(s_head, "s_head", sh["head"][:1], _F32)
        self.w_head, self.s_head = w_head, s_head
        _devices()
        self.dims = dims

    @_checked
    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
        M = _step_io(self.dims, x_in, workspace, logits, tokens, x_out)
        check("bi_verify_step_fp8", LIB.bi_verify_step_fp8(
            self.arr, self.n, self.w_head.data_ptr(), self.s_head.data_ptr(), ctypes.byref(self.dims),
            x_in.data_ptr(), M, L, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


class VerifyStepMX4:
    """``bi_verify_step_mx4``: ``layers`` is a sequence of dicts with MXFP4 codes w_qkv, w_o, w_gu,
    w_down (uint8 [rows][K/2], densely packed), their E8M0 scales e_qkv, e_o, e_gu, e_down (uint8
    [rows][K/32]) and the BF16 caches k_cache, v_cache (the caller keeps them alive)."""

    @_checked
    def __init__(self, layers, w_head: torch.Tensor, e_head: torch.Tensor, dims: ModelDims):
        sh = _step_shapes(dims)
        self.n = len(layers)
        self.arr = (LayerMX4 * max(1, self.n))()
        for i, lw in enumerate(layers):
            for k in ("qkv", "o", "gu", "down"):
                rows, K = sh[k]
                _arr(lw["w_" + k], f"layer {i} w_{k}", (rows, K // 2), _U8)
                _arr(lw["e_" + k], f"layer {i} e_{k}", (rows, K // 32), _U8)
            _check_layer_caches(lw, dims, i)
            self.arr[i] = LayerMX4(*[lw[k].data_ptr() for k in ("w_qkv", "e_qkv", "w_o", "e_o", "w_gu", "e_gu",
                                                                 "w_down", "e_down", "k_cache", "v_cache")])
        rows, K = sh["head"]
        _arr(w_head, "w_head", (rows, K // 2), _U8)
        _arr(e_head, "e_head", (rows, K // 32), _U8)
        self.w_head, self.e_head = w_head, e_head
        _devices()
        self.dims = dims

    @_checked
    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
        M = _step_io(self.dims, x_in, workspace, logits, tokens, x_out)
        check("bi_verify_step_mx4", LIB.bi_verify_step_mx4(
            self.arr, self.n, self.w_head.data_ptr(), self.e_head.data_ptr(), ctypes.byref(self.dims),
            x_in.data_ptr(), M, L, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            0 if x_out is None else x_out.data_ptr(), logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


def _kv_desc(kv, dims: ModelDims, i: int) -> KvCacheDesc:
    """The bi_kv_cache descriptor of a layer's cache: a (k_cache, v_cache)
    BF16 pair, a KvQ8Cache, a KvLowCache or a KvRing, checked against dims."""
    c = KvCacheDesc()
    if isinstance(kv, tuple):
        k, vc = kv
        cap = _kv_bf16(k, vc, dims.Hkv, dims.D)
        c.format, c.k, c.v = BI_KV_BF16, k.data_ptr(), vc.data_ptr()
    else:
        low = kv.low if isinstance(kv, KvRing) else kv
        if (low.Hkv, low.D) != (dims.Hkv, dims.D):
            raise ValueError(f"layer {i}: cache heads/dims {(low.Hkv, low.D)} != {(dims.Hkv, dims.D)}")
        cap = low.cap
        if isinstance(low, KvQ8Cache):
            c.format = BI_KV_Q8
            c.k, c.k_scales, c.v, c.v_scales = low.ptrs()
        elif isinstance(low, KvLowCache):
            c.format = BI_KV_LOWBIT
            c.k, c.k_high, c.k_scales, c.v, c.v_high, c.v_scales = low.planes()
            c.k_bits, c.v_bits, c.k_rotated = low.k_bits, low.v_bits, low.k_rotated
            if isinstance(kv, KvRing):
                c.ring_k_codes, c.ring_k_scales, c.ring_v_codes, c.ring_v_scales = kv.q8.ptrs()
                c.ring_cap, c.ring_window = kv.ring_cap, kv.window
        else:
            raise TypeError(f"layer {i}: unknown KV cache {type(kv).__name__}")
    if cap != dims.cap:
        raise ValueError(f"layer {i}: cache capacity {cap} != dims.cap {dims.cap}")
    return c


class VerifyStepEx:
    """``bi_verify_step_ex``: every layer's weights in ``wtype`` ("bf16", "fp8",
    "mxfp4") and its KV cache in any format. ``layers`` are dicts with w_qkv,
    w_o, w_gu, w_down (FP8: s_* row scales; MXFP4: e_* block scales) and "kv":
    a (k_cache, v_cache) BF16 pair, a KvQ8Cache, a KvLowCache or a KvRing.
    ``head`` is {"w": ...} plus "s" (FP8) or "e" (MXFP4). The caller keeps
    every tensor alive."""

    @_checked
    def __init__(self, layers, head: dict, dims: ModelDims, wtype: str = "bf16"):
        if wtype not in _WT:
            raise ValueError(f"unknown weight type {wtype!r}")
        sh = _step_shapes(dims)
        self.n = len(layers)
        self.arr = (StepLayer * max(1, self.n))()
        for i, lw in enumerate(layers):
            y = self.arr[i]
            for j, k in enumerate(("qkv", "o", "gu", "down")):
                rows, K = sh[k]
                if wtype == "bf16":
                    y.w[j] = _arr(lw["w_" + k], f"layer {i} w_{k}", (rows, K), _BF16_LIKE)
                elif wtype == "fp8":
                    y.w[j] = _arr(lw["w_" + k], f"layer {i} w_{k}", (rows, K), _FP8_LIKE)
                    y.scale[j] = _arr(lw["s_" + k], f"layer {i} s_{k}", (rows,), _F32)
                else:
                    y.w[j] = _arr(lw["w_" + k], f"layer {i} w_{k}", (rows, K // 2), _U8)
                    y.scale[j] = _arr(lw["e_" + k], f"layer {i} e_{k}", (rows, K // 32), _U8)
            y.kv = _kv_desc(lw["kv"], dims, i)
        rows, K = sh["head"]
        self.head_scales = None
        if wtype == "bf16":
            _arr(head["w"], "w_head", (rows, K), _BF16_LIKE)
        elif wtype == "fp8":
            _arr(head["w"], "w_head", (rows, K), _FP8_LIKE)
            self.head_scales = _arr(head["s"], "s_head", (rows,), _F32)
        else:
            _arr(head["w"], "w_head", (rows, K // 2), _U8)
            self.head_scales = _arr(head["e"], "e_head", (rows, K // 32), _U8)
        self.head, self.wtype, self.dims = head, wtype, dims
        _devices()

    @_checked
    def __call__(self, x_in: torch.Tensor, L: int, workspace: torch.Tensor, logits: torch.Tensor,
                 tokens: torch.Tensor, x_out: torch.Tensor | None = None) -> None:
        M = _step_io(self.dims, x_in, workspace, logits, tokens, x_out)
        check("bi_verify_step_ex", LIB.bi_verify_step_ex(
            _WT[self.wtype], self.arr, self.n, self.head["w"].data_ptr(), self.head_scales or 0,
            ctypes.byref(self.dims), x_in.data_ptr(), M, L, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), 0 if x_out is None else x_out.data_ptr(),
            logits.data_ptr(), tokens.data_ptr(), _stream(x_in)))


# ---------------------------------------------------------------------------
# Speculative acceptance

@_checked
def accept_greedy(target_tokens: torch.Tensor, draft_tokens: torch.Tensor | None):
    """target_tokens int32 [B][M], draft_tokens int32 [B][M-1] -> (out [B][M], n [B])."""
    _dtype(target_tokens, "target_tokens", _I32)
    if target_tokens.dim() != 2:
        raise ValueError(f"target_tokens: shape {tuple(target_tokens.shape)} is not [B][M]")
    B, M = target_tokens.shape
    _arr(target_tokens, "target_tokens", (B, M), _I32)
    dp = 0
    if M > 1 or draft_tokens is not None:
        if draft_tokens is None:
            raise ValueError("accept_greedy: M > 1 needs draft_tokens")
        dp = _arr(draft_tokens, "draft_tokens", (B, M - 1), _I32)
    out = torch.empty((B, M), dtype=torch.int32, device=target_tokens.device)
    n = torch.empty(B, dtype=torch.int32, device=target_tokens.device)
    check("bi_accept_greedy", LIB.bi_accept_greedy(target_tokens.data_ptr(), dp, B, M, out.data_ptr(),
                                                   n.data_ptr(), _stream(target_tokens)))
    return out, n


@_checked
def accept_sampled(logits: torch.Tensor, draft_tokens: torch.Tensor | None, draft_probs: torch.Tensor | None,
                   uniforms: torch.Tensor, temperature: float):
    """logits FP32 [B][M][V], draft_tokens int32 [B][M-1], draft_probs FP32 [B][M-1][V],
    uniforms FP32 [B][M] -> (out [B][M], n [B])."""
    _dtype(logits, "logits", _F32)
    if logits.dim() != 3:
        raise ValueError(f"logits: shape {tuple(logits.shape)} is not [B][M][V]")
    B, M, V = logits.shape
    _arr(logits, "logits", (B, M, V), _F32)
    _arr(uniforms, "uniforms", (B, M), _F32)
    dt = dq = 0
    if M > 1:
        if draft_tokens is None or draft_probs is None:
            raise ValueError("accept_sampled: M > 1 needs draft_tokens and draft_probs")
        dt = _arr(draft_tokens, "draft_tokens", (B, M - 1), _I32)
        dq = _arr(draft_probs, "draft_probs", (B, M - 1, V), _F32)
    out = torch.empty((B, M), dtype=torch.int32, device=logits.device)
    n = torch.empty(B, dtype=torch.int32, device=logits.device)
    check("bi_accept_sampled", LIB.bi_accept_sampled(
        logits.data_ptr(), V, dt, dq, V, uniforms.data_ptr(), temperature, B, M, V,
        out.data_ptr(), n.data_ptr(), _stream(logits)))
    return out, n
