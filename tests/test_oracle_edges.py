"""The oracle's quantizer on the edge-case groups that the GPU edge tests
feed through every plane writer (tests/_edges.py), pinned against exact
rational arithmetic: zero point = group minimum and step = range / (2^B - 1),
each rounded once to the nearest binary16 (ties to the even pattern); every
code the argmin over the 2^B levels of |x - (z + c s)|, exact ties to the
even code; a zero step gives code 0 ("Your KV Cache Doesn't Have a Bit
Problem...", section "What Quantization Error Is Actually Made Of", with the
readings where it is silent)."""
from fractions import Fraction

import numpy as np
import pytest

from _edges import edge_groups


def _half(bits):
    return Fraction(np.uint16(bits).view(np.float16).item())


def _rne16(fr):
    """Nearest binary16 bit pattern to a Fraction, ties to the even pattern,
    by search over the neighbours of the float64 estimate."""
    neg = fr < 0
    a = -fr if neg else fr
    lo = np.float16(float(a))
    with np.errstate(over="ignore"):  # the neighbour above 65504 is inf, dropped below
        cands = {int(np.float16(v).view(np.uint16)) for v in
                 (lo, np.nextafter(lo, np.float16(0)), np.nextafter(lo, np.float16(np.inf)))}
    cands = sorted(c for c in cands if c < 0x7C00)
    best = min(cands, key=lambda c: (abs(_half(c) - a), c % 2))
    return best | (0x8000 if neg and best != 0 else 0)


def _brute(x, bits):
    fx = [Fraction(float(v)) for v in x]
    mn, mx = min(fx), max(fx)
    # the zero point is the first minimal element: for a zero minimum that
    # element's sign of zero (a Fraction has none)
    first = next(v for v, f in zip(x, fx) if f == mn)
    z16 = _rne16(mn) | (0x8000 if mn == 0 and np.signbit(first) else 0)
    s16 = _rne16((mx - mn) / (2 ** bits - 1))
    z, s = _half(z16), _half(s16)
    codes = []
    for xi in fx:
        if s == 0:
            codes.append(0)
            continue
        codes.append(min((abs(xi - (z + c * s)), c % 2, c) for c in range(2 ** bits))[2])
    return codes, s16, z16


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_edge_groups_against_exact_arithmetic(orc, bits, dtype):
    names, groups = edge_groups(bits, dtype)
    for name, x in zip(names, groups):
        codes, s16, z16 = orc.quant_group(x.astype(np.float64), bits)
        want_codes, want_s, want_z = _brute(x, bits)
        assert z16 == want_z, f"{name}: zero {z16:#06x} != {want_z:#06x}"
        assert s16 == want_s, f"{name}: step {s16:#06x} != {want_s:#06x}"
        assert codes.tolist() == want_codes, f"{name}: codes differ"


def test_edge_groups_reach_the_corners(orc):
    """The constructed groups do contain what they are named for: exact ties
    of the quotient, zero steps from non-constant groups, subnormal steps and
    a binary16 rounding tie of the step itself."""
    seen = set()
    for bits in (2, 4, 8):
        for dtype in (np.float16, np.float32):
            names, groups = edge_groups(bits, dtype)
            for name, x in zip(names, groups):
                _, s16, z16 = orc.quant_group(x.astype(np.float64), bits)
                s, z = _half(s16), _half(z16)
                fx = [Fraction(float(v)) for v in x]
                if s != 0 and any(((xi - z) / s) % 1 == Fraction(1, 2) for xi in fx):
                    seen.add("tie")
                if s == 0 and max(fx) != min(fx):
                    seen.add("zero_step_nonconstant")
                if s16 != 0 and s16 < 0x0400:
                    seen.add("subnormal_step")
                exact = (max(fx) - min(fx)) / (2 ** bits - 1)
                for nb in (s16 - 1, s16 + 1):  # the step's binary16 neighbours
                    if 0 <= nb < 0x7C00 and exact - s == (_half(nb) - s) / 2:
                        seen.add("step_rounding_tie")
                if s16 == 0 and max(fx) == min(fx):
                    seen.add("zero_range")
                if np.dtype(dtype) == np.float32 and z != min(fx):
                    seen.add("f32_zero_not_min")
                if z16 == 0x8000:
                    seen.add("negative_zero_point")
    assert seen >= {"tie", "zero_step_nonconstant", "subnormal_step", "step_rounding_tie",
                    "zero_range", "f32_zero_not_min", "negative_zero_point"}, seen
