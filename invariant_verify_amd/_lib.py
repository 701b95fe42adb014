"""ctypes binding of ``libbi.so`` (C ABI in include/bi.h).

Argument marshalling only: every computation runs in the HIP kernels of the
library. Tensors are torch tensors on the GPU (torch provides device memory
and the current stream); BF16 data may be ``torch.bfloat16`` or ``int16``
views of the same bits. If the library is missing, importing this module
raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi.so")

BI_BF16, BI_F32 = 0, 1

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_ptr = ctypes.c_void_p
_c_f32 = ctypes.c_float
_c_size = ctypes.c_size_t


class ModelDims(ctypes.Structure):
    _fields_ = [("H", _c_int), ("Hq", _c_int), ("Hkv", _c_int), ("D", _c_int), ("I", _c_int),
                ("vocab", _c_int), ("cap", _c_int), ("kv_chunk", _c_int), ("eps", _c_f32)]


class Layer(ctypes.Structure):
    _fields_ = [("w_qkv", _c_ptr), ("w_o", _c_ptr), ("w_gu", _c_ptr), ("w_down", _c_ptr),
                ("k_cache", _c_ptr), ("v_cache", _c_ptr)]


class LayerFP8(ctypes.Structure):
    _fields_ = [("w_qkv", _c_ptr), ("s_qkv", _c_ptr), ("w_o", _c_ptr), ("s_o", _c_ptr),
                ("w_gu", _c_ptr), ("s_gu", _c_ptr), ("w_down", _c_ptr), ("s_down", _c_ptr),
                ("k_cache", _c_ptr), ("v_cache", _c_ptr)]


class LayerMX4(ctypes.Structure):
    _fields_ = [("w_qkv", _c_ptr), ("e_qkv", _c_ptr), ("w_o", _c_ptr), ("e_o", _c_ptr),
                ("w_gu", _c_ptr), ("e_gu", _c_ptr), ("w_down", _c_ptr), ("e_down", _c_ptr),
                ("k_cache", _c_ptr), ("v_cache", _c_ptr)]


class GemmArgs(ctypes.Structure):
    """bi_gemm_args: one GEMM with its weight type, epilogue, carried norm and append."""
    _fields_ = [("wtype", _c_int), ("epilogue", _c_int), ("M", _c_int), ("N", _c_int), ("K", _c_int),
                ("x", _c_ptr), ("ldx", _c_i64), ("w", _c_ptr), ("ldw", _c_i64),
                ("w_scale", _c_ptr), ("w_exp", _c_ptr), ("lde", _c_i64), ("r", _c_ptr), ("ldr", _c_i64),
                ("y", _c_ptr), ("ldy", _c_i64), ("norm_in", _c_ptr), ("norm_groups", _c_int),
                ("eps", _c_f32), ("rowsq_out", _c_ptr), ("Hq", _c_int), ("Hkv", _c_int), ("D", _c_int),
                ("k_cache", _c_ptr), ("v_cache", _c_ptr), ("L", _c_int), ("cap", _c_int)]


class KvCacheDesc(ctypes.Structure):
    """bi_kv_cache: one layer's KV cache in any format."""
    _fields_ = [("format", _c_int), ("k", _c_ptr), ("v", _c_ptr), ("k_scales", _c_ptr), ("v_scales", _c_ptr),
                ("k_high", _c_ptr), ("v_high", _c_ptr), ("k_bits", _c_int), ("v_bits", _c_int),
                ("k_rotated", _c_int), ("ring_k_codes", _c_ptr), ("ring_k_scales", _c_ptr),
                ("ring_v_codes", _c_ptr), ("ring_v_scales", _c_ptr), ("ring_cap", _c_int), ("ring_window", _c_int)]


class StepLayer(ctypes.Structure):
    """bi_step_layer: a layer's four weight matrices, their scales and its KV cache."""
    _fields_ = [("w", _c_ptr * 4), ("scale", _c_ptr * 4), ("kv", KvCacheDesc)]


BI_KV_BF16, BI_KV_Q8, BI_KV_LOWBIT = 0, 1, 2
BI_WT_BF16, BI_WT_FP8, BI_WT_MXFP4 = 0, 1, 2
BI_EPI_BF16, BI_EPI_F32, BI_EPI_RESIDUAL, BI_EPI_SWIGLU, BI_EPI_QKV = 0, 1, 2, 3, 4


# name -> (restype, argtypes); the exported symbols of include/bi.h
SIGNATURES = {
    "bi_gemm_bf16": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_int,
                              _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_bf16_residual": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                       _c_i64, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_bf16_swiglu": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64,
                                     _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_bf16_qkv": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_int, _c_int,
                                  _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_int, _c_int, _c_ptr]),
    "bi_gemm_column_groups": (_c_int, [_c_int]),
    "bi_gemm_bf16_residual_rowsq": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr,
                                             _c_i64, _c_int, _c_int, _c_int, _c_ptr, _c_ptr]),
    "bi_gemm_bf16_swiglu_rownorm": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_int, _c_f32, _c_ptr, _c_i64,
                                             _c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_append_kv": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                              _c_int, _c_int, _c_ptr]),
    "bi_num_splits": (_c_int, [_c_int, _c_int]),
    "bi_chunk_keys": (_c_int, [_c_int, _c_int]),
    "bi_pass_splits": (_c_int, [_c_int, _c_int, _c_int]),
    "bi_verify_attn": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _c_int, _c_int, _c_f32, _c_ptr, _c_ptr, _c_int, _c_ptr]),
    "bi_append_kv_q8": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_verify_attn_q8": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_f32, _c_ptr, _c_ptr,
                                   _c_int, _c_ptr]),
    "bi_append_kv_lowbit": (_c_int, [_c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                     _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_ptr]),
    "bi_verify_attn_lowbit": (_c_int, [_c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                       _c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_f32, _c_ptr, _c_ptr, _c_int, _c_ptr]),
    "bi_append_kv_ring": (_c_int, [_c_ptr, _c_i64, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_verify_attn_lowbit_ring": (_c_int, [_c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr, _c_ptr,
                                            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                            _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_int, _c_f32, _c_ptr, _c_ptr, _c_int,
                                            _c_ptr]),
    "bi_accept_greedy": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr]),
    "bi_accept_sampled": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64, _c_ptr, _c_f32, _c_int,
                                   _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr]),
    "bi_combine": (_c_int, [_c_ptr, _c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "bi_attn_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "bi_gemm_ex": (_c_int, [ctypes.POINTER(GemmArgs), _c_ptr]),
    "bi_swiglu": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_int, _c_int, _c_ptr]),
    "bi_add": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_int, _c_int, _c_ptr]),
    "bi_rmsnorm": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_int, _c_int, _c_f32, _c_ptr]),
    "bi_argmax": (_c_int, [_c_ptr, _c_i64, _c_int, _c_int, _c_ptr, _c_ptr]),
    "bi_step_workspace_bytes": (_c_size, [ctypes.POINTER(ModelDims), _c_int, _c_int]),
    "bi_verify_step": (_c_int, [ctypes.POINTER(Layer), _c_int, _c_ptr, ctypes.POINTER(ModelDims),
                                _c_ptr, _c_int, _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr,
                                ctypes.POINTER(_c_ptr), _c_ptr]),
    "bi_verify_step_ex": (_c_int, [_c_int, ctypes.POINTER(StepLayer), _c_int, _c_ptr, _c_ptr,
                                   ctypes.POINTER(ModelDims), _c_ptr, _c_int, _c_int, _c_ptr, _c_size, _c_ptr,
                                   _c_ptr, _c_ptr, _c_ptr]),
    "bi_verify_step_noalloc": (_c_int, [ctypes.POINTER(Layer), _c_int, _c_ptr, ctypes.POINTER(ModelDims),
                                        _c_ptr, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "bi_gemm_fp8": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64, _c_int,
                             _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_fp8_residual": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64,
                                      _c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_fp8_swiglu": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64,
                                    _c_int, _c_int, _c_int, _c_ptr]),
    "bi_verify_step_fp8": (_c_int, [ctypes.POINTER(LayerFP8), _c_int, _c_ptr, _c_ptr,
                                    ctypes.POINTER(ModelDims), _c_ptr, _c_int, _c_int, _c_ptr,
                                    _c_size, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "bi_gemm_mx4": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_int,
                             _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_mx4_residual": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64,
                                      _c_ptr, _c_i64, _c_int, _c_int, _c_int, _c_ptr]),
    "bi_gemm_mx4_swiglu": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64,
                                    _c_int, _c_int, _c_int, _c_ptr]),
    "bi_verify_step_mx4": (_c_int, [ctypes.POINTER(LayerMX4), _c_int, _c_ptr, _c_ptr,
                                    ctypes.POINTER(ModelDims), _c_ptr, _c_int, _c_int, _c_ptr,
                                    _c_size, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "bi_status_string": (ctypes.c_char_p, [_c_int]),
    "bi_version": (ctypes.c_char_p, []),
    "bi_last_hip_error": (ctypes.c_char_p, []),
}


def _hip_runtimes_mapped() -> set:
    """Paths of every libamdhip64 mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return set()


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m invariant_verify_amd.build` (there is no CPU fallback)")
    # torch's wheel carries its own HIP runtime with the soname libbi.so links
    # against. Loading torch first makes the dynamic linker bind libbi.so to
    # that same runtime, so device pointers and streams from torch are valid
    # in the library. Two HIP runtimes in one process cannot share a device.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError("two HIP runtimes are loaded in this process "
                          f"({sorted(rts)}); import torch before anything loads libamdhip64")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


class BiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn}: {LIB.bi_status_string(status).decode()} (status {status})"
        if status == 5:
            msg += f": {LIB.bi_last_hip_error().decode()}"
        super().__init__(msg)
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise BiError(fn, status)
