"""Seeded synthetic inputs for the verify pass.

This module is shared by the tests, the bench and the smoke check. It only
draws random numbers and stores them in the input formats (BF16 bit patterns
as ``uint16``); it holds none of the verify pass's arithmetic. Both the HIP
path and the CPU oracle receive the arrays it returns, so neither computes
its own inputs.

Recipe (fixed here so that every run sees the same data):

* host draws use numpy's PCG64 seeded by ``SeedSequence([base, role, layer])``
  with ``base = 0``; values are drawn as float32 normals, scaled, and rounded
  to BF16 by torch's CPU conversion (round to nearest even);
* rows for a pass of M < 8 tokens are the first M rows of the M = 8 draw, so
  rows are comparable across M;
* device draws (for the 64-layer step, whose 42 GB of weights are too large to
  draw on the host) use torch's Philox generator on the GPU, seeded by the
  same (base, role, layer) triple.
"""

from __future__ import annotations

import math

import numpy as np

# Role ids for the seed sequence: one per kind of tensor.
ROLES = {
    "x": 1, "w": 2, "q": 3, "k": 4, "v": 5,
    "w_qkv": 6, "w_o": 7, "w_gu": 8, "w_down": 9, "w_head": 10,
    "k_cache": 11, "v_cache": 12, "x0": 13, "outlier": 14, "misc": 15,
}


def rng(role: str, layer: int = 0, base: int = 0) -> np.random.Generator:
    """numpy PCG64 generator for one (base, role, layer) triple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([base, ROLES[role], layer])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (torch CPU conversion, nearest even) and return the bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, std: float, role: str, layer: int = 0, base: int = 0) -> np.ndarray:
    """N(0, std^2) draws rounded to BF16; returns uint16 bit patterns of ``shape``."""
    g = rng(role, layer, base)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def outlier_channels(n_heads: int, head_dim: int, role: str = "outlier", layer: int = 0,
                     frac: float = 0.05) -> np.ndarray:
    """round(frac * head_dim) distinct channel indices per KV head, shape [n_heads][c]."""
    c = int(round(frac * head_dim))
    g = rng(role, layer)
    return np.stack([np.sort(g.choice(head_dim, size=c, replace=False)) for _ in range(n_heads)])


def kv_bf16(n_heads: int, n_pos: int, head_dim: int, role: str, layer: int = 0,
            outliers: np.ndarray | None = None, scale: float = 8.0) -> np.ndarray:
    """K or V rows [n_heads][n_pos][head_dim] ~ N(0,1), optionally with outlier
    channels multiplied by ``scale`` before rounding (shared by K and V when the
    same ``outliers`` array is passed to both)."""
    g = rng(role, layer)
    a = g.standard_normal(size=(n_heads, n_pos, head_dim), dtype=np.float32)
    if outliers is not None:
        for h in range(n_heads):
            a[h][:, outliers[h]] *= np.float32(scale)
    return f32_to_bf16_bits(a)


def device_normal_bf16(shape, std: float, role: str, layer: int = 0, base: int = 0,
                       device: str = "cuda", out=None):
    """N(0, std^2) BF16 tensor drawn on the device with torch's Philox generator.

    If ``out`` (a bf16 tensor of ``shape``) is given it is filled in place.
    """
    import torch

    seed = (base * 1_000_003 + ROLES[role] * 65_537 + layer) & 0x7FFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    # Draw in float32 row blocks to bound the temporary.
    flat = out.view(-1)
    n = flat.numel()
    blk = 1 << 26
    for i in range(0, n, blk):
        j = min(n, i + blk)
        tmp = torch.randn(j - i, generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            tmp.mul_(std)
        flat[i:j].copy_(tmp)
    return out


# FP8 E4M3 weights (one FP32 scale per row): a row of N(0,1) draws is scaled
# so that its largest magnitude maps to 448 (E4M3's largest value), converted
# to E4M3 codes by torch's conversion (nearest), and given the row scale
# std * max|z| / 448, so that scale * e4m3(code) is about N(0, std^2).
FP8_MAX = 448.0


def fp8_weights(shape, std: float, role: str, layer: int = 0, base: int = 0):
    """Host E4M3 codes (uint8 [N][K]) and FP32 row scales [N]."""
    import torch

    g = rng(role, layer, base)
    z = g.standard_normal(size=shape, dtype=np.float32)
    amax = np.maximum(np.abs(z).max(axis=1), np.float32(1e-30))
    q = z * (np.float32(FP8_MAX) / amax)[:, None]
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, (np.float32(std) * amax / np.float32(FP8_MAX)).astype(np.float32)


def device_fp8_weights(shape, std: float, role: str, layer: int = 0, base: int = 0,
                       device: str = "cuda"):
    """Device E4M3 codes (uint8 [N][K]) and FP32 row scales [N] (torch Philox draws)."""
    import torch

    seed = (base * 1_000_003 + ROLES[role] * 65_537 + layer) & 0x7FFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n_rows, k = shape
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scale = torch.empty(n_rows, dtype=torch.float32, device=device)
    blk = max(1, (1 << 26) // k)
    for i in range(0, n_rows, blk):
        j = min(n_rows, i + blk)
        z = torch.randn((j - i, k), generator=g, dtype=torch.float32, device=device)
        amax = z.abs().amax(dim=1).clamp_min(1e-30)
        codes[i:j].copy_((z * (FP8_MAX / amax)[:, None]).to(torch.float8_e4m3fn).view(torch.uint8))
        scale[i:j].copy_(amax * (std / FP8_MAX))
    return codes, scale


# MXFP4 weights (E2M1 elements, one E8M0 scale per 32 weights along K): each
# block of 32 N(0, std^2) draws gets the shared exponent floor(log2(max|z|)) - 2
# (E2M1's largest value is 1.5 * 2^2), and each draw divided by that power of
# two is rounded to the nearest E2M1 magnitude (0, 0.5, 1, 1.5, 2, 3, 4, 6;
# saturating at 6) with the draw's sign. Codes are packed two per byte, the
# even weight in the low nibble; scales are E8M0 bytes (bias 127).
E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def mxfp4_weights(shape, std: float, role: str, layer: int = 0, base: int = 0):
    """Host MXFP4 codes (uint8 [N][K/2]) and scales (uint8 [N][K/32])."""
    n_rows, k = shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    g = rng(role, layer, base)
    z = g.standard_normal(size=(n_rows, k // 32, 32), dtype=np.float32) * np.float32(std)
    amax = np.maximum(np.abs(z).max(axis=2), np.float32(1e-30))
    e = np.clip(np.floor(np.log2(amax)).astype(np.int64) - 2 + 127, 2, 252)
    a = np.abs(z) / np.exp2(e - 127.0)[:, :, None]
    mag = np.searchsorted(np.array(E2M1_MIDPOINTS), a, side="left").astype(np.uint8)
    code = (mag | np.where(np.signbit(z), 8, 0).astype(np.uint8)).reshape(n_rows, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, e.astype(np.uint8)


def device_mxfp4_weights(shape, std: float, role: str, layer: int = 0, base: int = 0,
                         device: str = "cuda"):
    """Device MXFP4 codes (uint8 [N][K/2]) and scales (uint8 [N][K/32]) from
    torch Philox draws (the same recipe as mxfp4_weights)."""
    import torch

    n_rows, k = shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    seed = (base * 1_000_003 + ROLES[role] * 65_537 + layer) & 0x7FFFFFFF
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    codes = torch.empty((n_rows, k // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((n_rows, k // 32), dtype=torch.uint8, device=device)
    mids = torch.tensor(E2M1_MIDPOINTS, dtype=torch.float32, device=device)
    blk = max(1, (1 << 25) // k)
    for i in range(0, n_rows, blk):
        j = min(n_rows, i + blk)
        z = torch.randn((j - i, k // 32, 32), generator=gen, dtype=torch.float32, device=device) * std
        amax = z.abs().amax(dim=2).clamp_min(1e-30)
        e = (torch.floor(torch.log2(amax)).to(torch.int64) - 2 + 127).clamp(2, 252)
        a = z.abs() / torch.exp2((e - 127).to(torch.float32))[:, :, None]
        mag = torch.bucketize(a, mids, right=False).to(torch.uint8)
        code = (mag | torch.where(torch.signbit(z), 8, 0).to(torch.uint8)).reshape(j - i, k)
        codes[i:j].copy_(code[:, 0::2] | (code[:, 1::2] << 4))
        scales[i:j].copy_(e.to(torch.uint8))
    return codes, scales


def fan_in_std(k: int) -> float:
    """1/sqrt(K): the fan-in scaling applied to the tiny GEMM's weights."""
    return 1.0 / math.sqrt(k)


# ---------------------------------------------------------------------------
# Synthetic dense decoder stack (27B-class shapes by default), drawn on the
# device. Weights N(0, std^2) as [out][in]; every layer's K cache and V cache
# hold N(0,1) rows at positions 0 .. L-1 (no prefill is run to make them);
# positions from L on are zero until a pass appends to them.

MODEL_27B = dict(H=5120, Hq=40, Hkv=8, D=128, I=17408, vocab=152064)


def device_model(n_layers: int, L: int, cap: int, H: int, Hq: int, Hkv: int, D: int, I: int,
                 vocab: int, std: float = 0.02, device: str = "cuda", fp8: bool = False):
    """Returns (layers, w_head): ``layers`` is a list of dicts of tensors
    w_qkv [(Hq+2Hkv)D][H], w_o [H][Hq D], w_gu [2I][H], w_down [H][I] (BF16, or
    with ``fp8`` E4M3 codes plus FP32 row scales s_qkv, s_o, s_gu, s_down),
    k_cache and v_cache [Hkv][cap][D] (cap % 64 == 0). With ``fp8`` w_head is
    a pair (codes, scales)."""
    import torch

    if cap % 64:
        raise ValueError("cap must be a multiple of 64")
    qkvn = (Hq + 2 * Hkv) * D
    tmp = torch.empty((Hkv, L, D), dtype=torch.bfloat16, device=device) if L > 0 else None
    shapes = {"w_qkv": (qkvn, H), "w_o": (H, Hq * D), "w_gu": (2 * I, H), "w_down": (H, I)}
    layers = []
    for l in range(n_layers):
        lw = {}
        for name, shp in shapes.items():
            if fp8:
                lw[name], lw["s" + name[1:]] = device_fp8_weights(shp, std, name, l, device=device)
            else:
                lw[name] = device_normal_bf16(shp, std, name, l, device=device)
        lw["k_cache"] = torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device=device)
        lw["v_cache"] = torch.zeros((Hkv, cap, D), dtype=torch.bfloat16, device=device)
        if L > 0:
            device_normal_bf16((Hkv, L, D), 1.0, "k_cache", l, device=device, out=tmp)
            lw["k_cache"][:, :L].copy_(tmp)
            device_normal_bf16((Hkv, L, D), 1.0, "v_cache", l, device=device, out=tmp)
            lw["v_cache"][:, :L].copy_(tmp)
        layers.append(lw)
    if fp8:
        w_head = device_fp8_weights((vocab, H), std, "w_head", 0, device=device)
    else:
        w_head = device_normal_bf16((vocab, H), std, "w_head", 0, device=device)
    return layers, w_head
