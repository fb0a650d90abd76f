"""Pins for the oracle's binary16 conversions against the IEEE 754 format
definition and numpy's own binary16 routines (a library the oracle does not
use).  The stored step and zero point of every quantization group are
binary16, rounded once to nearest-even (reading taken where the pages say
only "fp16 metadata")."""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_half_to_double_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_double_to_half_roundtrip_exhaustive(orc):
    for b in range(65536):
        if (b & 0x7C00) == 0x7C00 and (b & 0x3FF):
            continue  # NaN payloads are not preserved
        x = orc.half_to_double(b)
        assert orc.double_to_half(x) == b, hex(b)


def test_midpoints_round_to_even(orc):
    # Between consecutive positive halves a < b, the exact midpoint (exact in
    # double) rounds to the one with the even bit pattern; just below / above
    # it rounds down / up.
    for h in range(0, 0x7BFF):
        a = orc.half_to_double(h)
        b = orc.half_to_double(h + 1)
        m = (a + b) / 2
        even = h if h % 2 == 0 else h + 1
        assert orc.double_to_half(m) == even, hex(h)
        assert orc.double_to_half(np.nextafter(m, -np.inf)) == h
        assert orc.double_to_half(np.nextafter(m, np.inf)) == h + 1
        assert orc.double_to_half(-m) == even | 0x8000
    # 65520 is the midpoint between 65504 and the (infinite) next binade.
    assert orc.double_to_half(65520.0) == 0x7C00
    assert orc.double_to_half(np.nextafter(65520.0, 0)) == 0x7BFF
    assert orc.double_to_half(1e300) == 0x7C00
    # below half the smallest subnormal: zero; above it: the subnormal
    assert orc.double_to_half(2.0 ** -26) == 0
    assert orc.double_to_half(2.0 ** -25) == 0       # tie -> even (0)
    assert orc.double_to_half(np.nextafter(2.0 ** -25, 1)) == 1
    assert orc.double_to_half(3 * 2.0 ** -25) == 2   # tie 1|2 -> even 2


def test_double_to_half_matches_numpy_random(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(40000) * 10.0 ** rng.integers(-9, 5, 40000),
        rng.uniform(-70000, 70000, 5000),
        rng.uniform(0, 2.0 ** -13, 5000),
    ])
    ref = x.astype(np.float16).view(np.uint16)  # numpy: double -> half directly
    got = np.array([orc.double_to_half(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
