"""Pins of the oracle's bf16 conversions (oracle/bf16.py).

Every pool byte and every Q/K/V input reaches the oracle's float64 arithmetic
through bf16_bits_to_f64, so a slip there (a widening that loses the high
bits, a wrong shift, the pattern read as float16) would sit on both sides of
every CPU comparison that goes through bit patterns.  These tests fix it to
values that do not come from the oracle: hand-typed bf16 patterns with their
IEEE-754 values (a bf16 value is the upper half of a binary32 value: 1 sign
bit, 8 exponent bits with bias 127, 7 fraction bits), and torch's own
bfloat16 -> float64 conversion over all 65,536 patterns.  The narrowing
direction, used to build test inputs, is pinned on round-to-nearest,
ties-to-even cases worked out by hand.

The pools hold bf16 ("How to Improve Streaming Inference Performance with
FlashInfer KV Cache Backend", section "Force-FP32 Fallback Avoidance": the
pages keep K/V in bf16 and warn against a float32 path).
"""

import math

import numpy as np
import pytest
import torch

import oracle.bf16 as bf16

# (pattern, value) typed by hand from the bf16 format
HAND = [
    (0x3F80, 1.0),                        # exponent 127, fraction 0
    (0xC000, -2.0),                       # sign 1, exponent 128
    (0x0000, 0.0),
    (0x4049, 3.140625),                   # 2 * (1 + 73/128)
    (0x3E80, 0.25),                       # exponent 125
    (0x3FC0, 1.5),                        # fraction 0b1000000
    (0x0001, 2.0 ** -133),                # smallest subnormal: 2^-126 * 2^-7
    (0x0080, 2.0 ** -126),                # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite, 3.3895e38
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x4300, 128.0),
    (0xBF01, -(1.0 + 1.0 / 128) * 0.5),   # exponent 126, fraction 1
]


@pytest.mark.parametrize("bits,value", HAND)
def test_widening_hand_values(bits, value):
    got = bf16.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))
    assert got.dtype == np.float64
    assert got[0] == value


def test_widening_signed_zero_and_infinities():
    got = bf16.bf16_bits_to_f64(np.array([0x8000, 0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) == -1.0
    assert got[1] == math.inf and got[2] == -math.inf
    assert math.isnan(got[3])


def test_widening_every_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns
        ours = bf16.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # and sign bits agree (for the zeros too)
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_widening_keeps_shape():
    b = np.array([[0x3F80, 0x4000], [0xC040, 0x0000]], dtype=np.uint16)
    assert np.array_equal(bf16.bf16_bits_to_f64(b), [[1.0, 2.0], [-3.0, 0.0]])


# (value, expected pattern): round to nearest, ties to even, worked by hand.
# The spacing of bf16 in [1, 2) is 2^-7.
NARROW = [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie between 0x3F80 and 0x3F81: even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie between 0x3F81 and 0x3F82: even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie: up
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),    # just below the tie: down
    (-1.0 - 3 * 2.0 ** -8, 0xBF82),
    (2.0 - 2.0 ** -9, 0x4000),                 # tie at the top of the binade: to 2.0
    (0.25, 0x3E80),
    (-2.0, 0xC000),
    (0.0, 0x0000),
]


@pytest.mark.parametrize("value,bits", NARROW)
def test_narrowing_rounds_to_nearest_even(value, bits):
    assert int(bf16.f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_narrowing_round_trip_of_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        x = bf16.bf16_bits_to_f64(bits)
    keep = np.isfinite(x)
    back = bf16.f64_to_bf16_bits(x[keep])
    assert np.array_equal(back, bits[keep])
