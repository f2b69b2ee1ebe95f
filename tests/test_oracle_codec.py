"""Pins of the oracle's fp16/bf16 decoder and round-to-nearest-even encoder.

Every check is against something other than the oracle's own formula: numpy's
IEEE binary16 type, the bfloat16 definition as the upper half of a binary32
(numpy bit reinterpretation), torch's float32 -> bfloat16 conversion, and
hand-worked boundary values of the formats.
"""
import numpy as np
import pytest
import torch

from oracle import oracle

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_decode_f16_exhaustive_vs_numpy():
    got = oracle.decode(ALL, "f16")
    ref = ALL.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive_vs_upper_half_of_binary32():
    with np.errstate(invalid="ignore"):
        ref = (ALL.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.decode(ALL, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_encode_roundtrips_every_finite_pattern(fmt):
    vals = oracle.decode(ALL, fmt)
    finite = np.isfinite(vals)
    back = oracle.encode(vals[finite], fmt)
    assert np.array_equal(back, ALL[finite])


def test_encode_f16_random_doubles_vs_numpy():
    rng = np.random.default_rng(7)
    # wide dynamic range incl. subnormals, overflow and exact ties
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 20, 200_000))
    ties = (np.arange(-4096, 4096) + 0.5) * np.exp2(-8)  # midpoints at 2^-8 spacing
    x = np.concatenate([x, ties, -x[:1000]])
    got = oracle.encode(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_encode_bf16_vs_torch_on_binary32_values():
    # Doubles that are exact binary32 values, so torch's float32 -> bf16
    # conversion is a single rounding of the same value.
    rng = np.random.default_rng(8)
    x32 = (rng.standard_normal(200_000) * np.exp2(rng.integers(-140, 120, 200_000))).astype(np.float32)
    special = np.array([np.finfo(np.float32).max, np.finfo(np.float32).tiny,
                        1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                        -(1.0 + 2.0 ** -8), 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135], dtype=np.float32)
    x32 = np.concatenate([x32, special])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_encode_boundaries_hand_worked():
    f16 = lambda v: int(oracle.encode(np.array([v]), "f16")[0])
    bf16 = lambda v: int(oracle.encode(np.array([v]), "bf16")[0])
    assert f16(65504.0) == 0x7BFF          # largest finite
    assert f16(65519.99) == 0x7BFF         # below the overflow midpoint
    assert f16(65520.0) == 0x7C00          # midpoint ties away to infinity (even = inf)
    assert f16(2.0 ** -24) == 0x0001       # smallest subnormal
    assert f16(2.0 ** -25) == 0x0000       # half of it: tie to even (zero)
    assert f16(3 * 2.0 ** -25) == 0x0002   # 1.5 ulp: tie to even (2)
    assert f16(2049.0) == 0x6800           # 2049 is a tie between 2048 and 2050 -> 2048
    assert f16(2051.0) == 0x6802           # tie between 2050 and 2052 -> 2052
    assert f16(-0.0) == 0x8000
    assert f16(float("inf")) == 0x7C00
    assert bf16(1.0) == 0x3F80
    assert bf16(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    assert bf16(-2.0) == 0xC000
