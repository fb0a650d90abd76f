"""Pins for the oracle's quantizer and packing.

What the pages fix ("Your KV Cache Doesn't Have a Bit Problem...", section
"What Quantization Error Is Actually Made Of"): zero point = group minimum,
step = range / (2^B - 1), every element rounded to the nearest step, so the
error per element is at most half a step and 2^B levels exist.  The checks
below use exact rational arithmetic (fractions) and closed forms, not the
oracle's own fp64 formula."""
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked.txt")


def _parse_values(spec):
    out = []
    for tok in spec.split():
        if "*" in tok:
            v, k = tok.split("*")
            out += [float(v)] * int(k)
        else:
            out.append(float(tok))
    return out


def _golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, bits, vals, meta, words = [f.strip() for f in line.split("|")]
        cases.append((name, int(bits), _parse_values(vals), int(meta, 16),
                      None if words == "-" else [int(w, 16) for w in words.split()]))
    return cases


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c[0])
def test_golden_worked_groups(orc, case):
    name, bits, vals, meta, words = case
    assert len(vals) == 32
    codes, s16, z16 = orc.quant_group(np.array(vals), bits)
    assert (s16 | (z16 << 16)) == meta
    if words is not None:
        assert orc.pack(codes, bits).tolist() == words
    if name == "tie_b2":
        assert codes[:6].tolist() == [0, 3, 0, 2, 2, 1]


def test_pack_closed_forms(orc):
    j = np.arange(32)
    assert orc.pack(j % 4, 2).tolist() == [0xE4E4E4E4] * 2
    assert orc.pack(j % 16, 4).tolist() == [0x76543210, 0xFEDCBA98] * 2
    w8 = orc.pack(j, 8).tolist()
    assert w8[0] == 0x03020100 and w8[1] == 0x07060504 and w8[7] == 0x1F1E1D1C
    rng = np.random.default_rng(0)
    for bits in (1, 2, 4, 8):
        c = rng.integers(0, 2 ** bits, 64).astype(np.uint8)
        assert np.array_equal(orc.unpack(orc.pack(c, bits), 64, bits), c)


def _h(bits):
    return Fraction(np.uint16(bits).view(np.float16).item())


def _exact_round_half(fr):
    """Nearest binary16 to a non-negative Fraction, ties to even bit pattern
    (brute force over the two neighbouring representable values)."""
    f = float(fr)
    lo = np.float16(f)
    cands = {int(np.float16(v).view(np.uint16)) for v in
             (lo, np.nextafter(lo, np.float16(0)), np.nextafter(lo, np.float16(np.inf)))}
    cands = sorted(c for c in cands if c < 0x7C00)
    best = min(cands, key=lambda c: (abs(_h(c) - fr), c % 2))
    return best


def _brute_codes(x, s, z, bits):
    """argmin over all 2^B levels of |x - (z + c*s)| exactly; exact ties go
    to the even code."""
    out = []
    for xi in x:
        fx = Fraction(float(xi))
        if s == 0:
            out.append(0)
            continue
        errs = [(abs(fx - (z + c * s)), c % 2, c) for c in range(2 ** bits)]
        out.append(min(errs)[2])
    return out


def _groups(rng, n_groups, scale_pow=(-3, 3)):
    gs = []
    for _ in range(n_groups):
        sc = 10.0 ** rng.uniform(*scale_pow)
        x = (rng.standard_normal(32) * sc).astype(np.float16)
        if rng.random() < 0.3:  # an outlier inflates the step
            x[rng.integers(32)] *= np.float16(40)
        gs.append(x)
    return gs


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_brute_force_nearest_level_and_step(orc, bits):
    rng = np.random.default_rng(10 + bits)
    for x in _groups(rng, 60):
        codes, s16, z16 = orc.quant_group(x.astype(np.float64), bits)
        fx = [Fraction(float(v)) for v in x]
        mn, mx = min(fx), max(fx)
        assert z16 == _exact_round_half(mn) if mn >= 0 else True
        assert _h(z16) == mn  # binary16 inputs: the zero point is the minimum
        assert s16 == _exact_round_half((mx - mn) / (2 ** bits - 1))
        assert codes.tolist() == _brute_codes(x, _h(s16), _h(z16), bits)


def test_exact_ties_go_to_even(orc):
    # Elements placed exactly half-way between levels.
    rng = np.random.default_rng(3)
    checked = 0
    for bits in (2, 4):
        for _ in range(200):
            z = float(np.float16(rng.uniform(-4, 4)))
            s = float(np.float16(2.0 ** rng.integers(-6, 2)))
            top = 2 ** bits - 1
            x = [z, z + top * s] + [z + (k + 0.5) * s for k in rng.integers(0, top, 30)]
            x = np.array(x)
            if not np.array_equal(x.astype(np.float16).astype(np.float64), x):
                continue  # only groups whose tie points are binary16 values
            codes, s16, z16 = orc.quant_group(x, bits)
            assert _h(s16) == Fraction(s) and _h(z16) == Fraction(z)
            for xi, c in zip(x[2:], codes[2:]):
                k = int(round((xi - z) / s - 0.5))
                assert c == (k if k % 2 == 0 else k + 1)
            checked += 1
    assert checked >= 50


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_error_bound_range_and_extremes(orc, bits):
    """|x - xhat| <= step/2 exactly, codes in [0, 2^B-1], the minimum gets
    code 0 and the maximum code 2^B-1 (binary16 inputs, normal step)."""
    rng = np.random.default_rng(100 + bits)
    k = rng.standard_normal((4, 64, 32)).astype(np.float16)
    k[:, 5, :] *= np.float16(60)
    for x in k.reshape(-1, 32):
        codes, s16, z16 = orc.quant_group(x.astype(np.float64), bits)
        s, z = _h(s16), _h(z16)
        assert codes.max() <= 2 ** bits - 1
        normal = (s16 & 0x7C00) != 0
        for xi, c in zip(x, codes):
            err = abs(Fraction(float(xi)) - (z + c * s))
            if normal:
                assert err <= s / 2
            else:
                assert err <= Fraction(float(x.max())) - Fraction(float(x.min()))
        if normal:
            assert codes[np.argmin(x)] == 0
            assert codes[np.argmax(x)] == 2 ** bits - 1


def test_zero_range_groups_exact(orc):
    for v in (1.25, -3.0, 0.0, 6.1035156e-05, 65504.0):
        x = np.full(32, np.float16(v), dtype=np.float64)
        codes, s16, z16 = orc.quant_group(x, 2)
        assert s16 == 0 and codes.max() == 0 and _h(z16) == Fraction(float(np.float16(v)))


def test_fp32_inputs_bound_with_zero_slack(orc):
    """fp32 inputs (the tiny workload): the zero point is the minimum rounded
    to binary16, so the bound gains |min - zero|."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        x = rng.standard_normal(32).astype(np.float32)
        x[3] *= 50
        codes, s16, z16 = orc.quant_group(x.astype(np.float64), 2)
        s, z = _h(s16), _h(z16)
        slack = abs(Fraction(float(x.min())) - z)
        for xi, c in zip(x, codes):
            assert abs(Fraction(float(xi)) - (z + c * s)) <= s / 2 + slack
        assert codes.max() <= 3


def test_key_planes_group_per_channel_and_tail(orc):
    """Keys: one group = one channel over G consecutive tokens; tokens past
    the last full group are copied verbatim into the tail."""
    rng = np.random.default_rng(5)
    nb, h, T, D, G = 2, 3, 75, 64, 32
    k = rng.standard_normal((nb, h, T, D)).astype(np.float16)
    kc, km, kt = orc.quantize_keys(k, 2, G, max_tokens=96)
    assert kc.shape == (nb, h, 3, D, 2) and km.shape == (nb, h, 3, D)
    for b, hh, g, c in [(0, 0, 0, 0), (1, 2, 1, 63), (0, 1, 1, 17)]:
        codes, s16, z16 = orc.quant_group(k[b, hh, g * G:(g + 1) * G, c].astype(np.float64), 2)
        assert km[b, hh, g, c] == (s16 | (z16 << 16))
        assert np.array_equal(kc[b, hh, g, c], orc.pack(codes, 2))
    assert np.all(km[:, :, 2] == 0)           # group 2 not full: untouched
    assert np.array_equal(kt[:, :, :T - 64], k[:, :, 64:])


def test_value_planes_group_per_token(orc):
    rng = np.random.default_rng(6)
    nb, h, T, D, G = 1, 2, 40, 128, 32
    v = rng.standard_normal((nb, h, T, D)).astype(np.float16)
    vc, vm = orc.quantize_values(v, 4, G, max_tokens=64)
    assert vc.shape == (nb, h, 64, 4, 4)
    for hh, t, cg in [(0, 0, 0), (1, 39, 3), (0, 17, 2)]:
        codes, s16, z16 = orc.quant_group(v[0, hh, t, cg * G:(cg + 1) * G].astype(np.float64), 4)
        assert vm[0, hh, t, cg] == (s16 | (z16 << 16))
        assert np.array_equal(vc[0, hh, t, cg], orc.pack(codes, 4))
