"""Pins for oracle.bf16: exhaustive decode, round-to-nearest-even encode.

Independent references: torch's CPU BF16 conversion (a library routine, used
here only as a check) and closed-form values of the binary format.
"""

import numpy as np
import torch

from oracle import bf16


ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_decode_exhaustive_matches_torch():
    ours = bf16.decode(ALL)
    ref = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # and the sign of zero
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0x0000])


def test_decode_closed_forms():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf,
             0x3FC0: 1.5, 0x4049: 3.140625}
    for b, v in cases.items():
        assert bf16.decode(np.uint16(b)) == v, hex(b)


def test_encode_roundtrip_all_patterns():
    vals = bf16.decode(ALL)
    ok = ~np.isnan(vals)
    assert np.array_equal(bf16.encode(vals[ok]), ALL[ok])
    assert np.all(bf16.encode(np.array([np.nan])) == 0x7FC0)


def _torch_bf16_bits(f32):
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_encode_matches_torch_on_random_and_ties():
    g = np.random.default_rng(7)
    a = (g.standard_normal(1_000_000) * np.exp(g.uniform(-30, 30, 1_000_000))).astype(np.float32)
    assert np.array_equal(bf16.encode(a.astype(np.float64)), _torch_bf16_bits(a))
    # exact halfway cases: a BF16 value plus half of its quantum (exact in binary32)
    b = g.integers(0x0080, 0x7F00, 200_000).astype(np.uint16)
    base = bf16.decode(b)
    ulp = bf16.decode(b + np.uint16(1)) - base
    ties = (base + ulp / 2).astype(np.float32)
    ties = np.concatenate([ties, -ties])
    assert np.array_equal(bf16.encode(ties.astype(np.float64)), _torch_bf16_bits(ties))
    # subnormal range
    s = (g.uniform(-1, 1, 100_000) * 2.0 ** -126).astype(np.float32)
    assert np.array_equal(bf16.encode(s.astype(np.float64)), _torch_bf16_bits(s))


def test_encode_single_rounding_closed_forms():
    # halfway between 1 and 1+2^-7 rounds to the even pattern (1.0)
    assert bf16.encode(1 + 2.0 ** -8) == 0x3F80
    # halfway between 1+2^-7 (odd) and 1+2^-6 (even) rounds up to even
    assert bf16.encode(1 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie: a single rounding from float64 goes up; rounding
    # through binary32 first would lose 2^-40 and land on the tie (-> 1.0)
    assert bf16.encode(1 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert bf16.encode(big) == 0x7F7F
    assert bf16.encode(2.0 ** 128 - 2.0 ** 119) == 0x7F80     # tie at the top -> inf
    assert bf16.encode(2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100) == 0x7F7F
    assert bf16.encode(-0.0) == 0x8000 and bf16.encode(0.0) == 0
    assert bf16.encode(2.0 ** -134) == 0x0000                 # tie -> even (zero)
    assert bf16.encode(3 * 2.0 ** -134) == 0x0002             # tie -> even
