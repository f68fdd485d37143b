"""Pins for the oracle's binary16 codec.

The codec is checked against numpy's own float16 conversions (a library
routine: exact widening, and correctly rounded round-to-nearest-even
narrowing), exhaustively for decoding and on a million drawn doubles plus
every tie point for encoding, and against values fixed by the IEEE-754
binary16 format itself.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore:overflow")


def test_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros survive
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_encode_roundtrips_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    back = oracle.f16_encode(vals[finite])
    assert np.array_equal(back, bits[finite])
    # infinities keep their sign, NaN becomes a NaN pattern
    assert oracle.f16_encode(np.array([np.inf, -np.inf])).tolist() == [0x7C00, 0xFC00]
    n = oracle.f16_encode(np.array([np.nan]))[0]
    assert (n & 0x7C00) == 0x7C00 and (n & 0x03FF) != 0


def test_encode_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(1234)
    mag = np.exp2(rng.uniform(-30, 17, size=1_000_000))
    x = mag * rng.choice([-1.0, 1.0], size=mag.size)
    ours = oracle.f16_encode(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_ties_and_neighbours_match_numpy():
    # midpoints between every pair of adjacent positive finite fp16 values,
    # and the doubles just below / above each midpoint
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2  # exact in double
    for x in (mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)):
        for sgn in (1.0, -1.0):
            v = sgn * x
            assert np.array_equal(oracle.f16_encode(v), v.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (2.0 ** -24, 0x0001),
    (2.0 ** -14, 0x0400), (0.5, 0x3800), (0.0, 0x0000), (-0.0, 0x8000),
    # ties go to the even neighbour
    (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
    (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
    # overflow threshold: 65520 is the midpoint between 65504 and 2^16
    (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e6, 0x7C00),
    # the largest subnormal rounds up into the smallest normal
    (2.0 ** -14 - 2.0 ** -26, 0x0400),
])
def test_encode_format_fixed_points(x, bits):
    """Values fixed by the binary16 layout: 1 sign, 5 exponent (bias 15), 10 fraction bits."""
    assert int(oracle.f16_encode(np.array([x]))[0]) == bits
