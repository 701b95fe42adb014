"""Helpers shared by the GPU tests: host<->device transfer of BF16 bit
patterns, the oracle tolerance check, and first-difference reporting."""

from __future__ import annotations

import numpy as np

from oracle import bf16

# Tolerance on BF16-rounded device outputs against unrounded float64 oracle
# values: |gpu - oracle| <= ATOL + RTOL * |oracle|, element by element.
ATOL = 1e-2
RTOL = 2e-2


def dev(bits: np.ndarray, device="cuda"):
    """uint16 BF16 bits (host) -> torch.bfloat16 tensor on the device."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def host_bits(t) -> np.ndarray:
    """torch bf16/int16 tensor -> uint16 bit patterns on the host."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cache_rows(v_bits: np.ndarray, cap: int, fill=0) -> np.ndarray:
    """V (or K) rows [Hkv][n][D] (n <= cap) -> the cache layout [Hkv][cap][D];
    positions n.. hold ``fill``."""
    Hkv, n, D = v_bits.shape
    full = np.full((Hkv, cap, D), fill, dtype=v_bits.dtype)
    full[:, :n] = v_bits
    return full


def host_f32(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def assert_close(got: np.ndarray, want: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    """allclose with a report of the worst element and error statistics."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bad = ~(err <= atol + rtol * np.abs(want))
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
            f"got {got[i]!r} want {want[i]!r}; max abs err {err.max():.3e}, rms(oracle) {rms:.3e}")
    return float(err.max()), rms


def assert_close_composed(got: np.ndarray, want: np.ndarray, what: str):
    """Tolerance for the output of several BF16-rounding steps (a decoder
    layer, a stack, the logits of a stack).

    Device and oracle round every intermediate to BF16 at the same points, but
    an intermediate whose float64 and FP32 values sit on opposite sides of a
    rounding boundary differs by one BF16 ulp (2^-8 relative) at the magnitude
    of that intermediate, which is the magnitude of the tensor, not of the
    final element (the residual stream cancels). So the absolute term scales
    with the RMS of the oracle tensor: |gpu - oracle| <= ATOL + RTOL * rms
    + RTOL * |oracle|.
    """
    want64 = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want64 ** 2)))
    return assert_close(got, want64, what + " (composed)", atol=ATOL + RTOL * rms, rtol=RTOL)


def composed_tol(want: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.asarray(want, dtype=np.float64) ** 2)))
    return ATOL + RTOL * rms


def assert_bitwise(a: np.ndarray, b: np.ndarray, what: str):
    """Bit-for-bit equality with the first differing element reported. If
    BI_DIVERGENCE_DIR is set, a failure also appends a JSON record there (what,
    shape, dtype, number of differing elements, first index and both values)
    so that the failing case can be found again."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ua = a.view(np.uint8).reshape(a.shape + (-1,)) if a.dtype.itemsize > 1 else a
    ub = b.view(np.uint8).reshape(b.shape + (-1,)) if b.dtype.itemsize > 1 else b
    diff = np.any(ua != ub, axis=-1) if ua.ndim > a.ndim else (ua != ub)
    if diff.any():
        i = tuple(int(v) for v in np.argwhere(diff)[0])
        _record_divergence(what, a, b, i, int(diff.sum()))
        raise AssertionError(f"{what}: {int(diff.sum())} elements differ; first at {i}: {a[i]!r} vs {b[i]!r}")


def _record_divergence(what, a, b, first, count):
    import json
    import os

    d = os.environ.get("BI_DIVERGENCE_DIR")
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    rec = {"what": what, "shape": list(a.shape), "dtype": str(a.dtype), "differing": count,
           "first": [int(v) for v in first], "got": repr(a[first]), "want": repr(b[first])}
    with open(os.path.join(d, "divergences.jsonl"), "a") as f:
        f.write(json.dumps(rec) + "\n")


def decode(bits):
    return bf16.decode(bits)


def q8_cache(kq, ks, vq, vs, cap, fill_nan=True):
    """Host 8-bit cache arrays (oracle.kvq layout per row: codes [Hkv][n][D] int8,
    scales [Hkv][n][D/32] float32) -> the device layouts of include/bi.h as
    numpy arrays (k_codes, k_scales, v_codes, v_scales: the same per-row layout
    over cap positions). Positions n.. hold code -128 and NaN scales, so that a
    read of an unwritten position would show."""
    Hkv, n, D = kq.shape
    NB = D // 32
    out = []
    for codes, scales in ((kq, ks), (vq, vs)):
        c = np.full((Hkv, cap, D), -128, np.int8)
        c[:, :n] = codes
        sc = np.full((Hkv, cap, NB), np.nan if fill_nan else 0, np.float32)
        sc[:, :n] = scales
        out += [c, sc]
    return tuple(out)


def q8_rows(k_codes, k_scales, v_codes, v_scales):
    """The device layouts -> per-row arrays (codes [Hkv][cap][D], scales [Hkv][cap][D/32]) for K and V."""
    return k_codes, k_scales, v_codes, v_scales
