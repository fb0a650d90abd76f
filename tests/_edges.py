"""Quantizer edge-case inputs: 32-value groups built to hit the corners of
the quantizer's definition (zero point = group minimum, step = range /
(2^B - 1), nearest step; "Your KV Cache Doesn't Have a Bit Problem...",
section "What Quantization Error Is Actually Made Of"), with the readings
taken where the page is silent (binary16 step and zero rounded once, exact
ties to the even code, zero step -> code 0).

Inputs only: every expected value comes from the oracle.  The groups are
tiled into key tensors (a group runs down one channel over 32 tokens) and
value tensors (a group runs along 32 channels of one token) so that every
quantized group of a small cache is one of them.
"""
from __future__ import annotations

import os

import numpy as np

G = 32
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_worked.txt")


def _exact(vals, dtype):
    """vals (float64) as `dtype`, asserting that each value is exact (signs of
    zero included)."""
    a = np.asarray(vals, dtype=np.float64)
    b = a.astype(dtype)
    assert np.array_equal(b.astype(np.float64), a) and \
        np.array_equal(np.signbit(b), np.signbit(a)), f"not exact in {np.dtype(dtype)}: {a}"
    return b


def golden_groups():
    """The hand-worked groups of tests/golden/quant_worked.txt (inputs only)."""
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, _bits, inputs, _meta, _words = [s.strip() for s in line.split("|")]
            xs = []
            for tok in inputs.split():
                if "*" in tok:
                    v, k = tok.split("*")
                    xs += [float(v)] * int(k)
                else:
                    xs.append(float(tok))
            assert len(xs) == G, name
            out.append((name, np.array(xs)))
    return out


def _fill(core, filler):
    """A 32-value group: the listed values, then `filler` values cycling."""
    core = list(core)
    while len(core) < G:
        core.append(filler[(len(core)) % len(filler)])
    return core[:G]


def edge_groups(bits: int, dtype=np.float16, seed: int = 0):
    """(names, array [N][32] of dtype) of edge-case groups for B = bits."""
    top = (1 << bits) - 1
    rng = np.random.default_rng(seed)
    names, groups = [], []

    def add(name, vals):
        names.append(name)
        groups.append(_exact(vals, dtype))

    for name, xs in golden_groups():
        add("golden_" + name, xs)

    # zero range: one constant (the step is 0, every code 0)
    for c in (0.0, 1.25, -3.5, 65504.0, -65504.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -14,
              0.0009765625, 1000.0):
        add(f"const_{c}", [c] * G)

    # exact ties: zero point z, step s exactly representable, elements at
    # z + (k + 1/2) s for k = 0 .. top - 1 (both neighbours of each tie
    # present through z and z + top * s)
    for z, s in ((0.0, 1.0), (-2.0, 0.5), (3.0, 0.25), (-1.5, 0.75), (100.0, 0.125),
                 (-0.001953125, 2.0 ** -12)):
        ks = [(i * 37) % top for i in range(G - 2)]
        vals = [z, z + top * s] + [z + (k + 0.5) * s for k in ks]
        if np.array_equal(np.asarray(vals).astype(dtype).astype(np.float64), vals):
            add(f"ties_z{z}_s{s}", vals)  # only where every tie is on the input grid

    # near ties: a few binary16 ulps either side of each tie (z = 0, s = 1
    # and z = -2, s = 0.5)
    for z, s in ((0.0, 1.0), (-2.0, 0.5)):
        vals = [z, z + top * s]
        k = 0
        while len(vals) < G:
            t = z + ((k % top) + 0.5) * s
            th = np.float16(t)
            for m in (1, 2, 3):
                up, dn = th, th
                for _ in range(m):
                    up = np.nextafter(up, np.float16(np.inf))
                    dn = np.nextafter(dn, np.float16(-np.inf))
                vals += [float(up), float(dn)]
            k += 1
        add(f"near_ties_z{z}_s{s}", vals[:G])

    # the binary16 step itself a rounding tie: range / top exactly halfway
    # between two binary16 values (1 and 1 + 2^-10), so it goes to even (1)
    if bits == 2:
        add("step_tie_even", _fill([-3 * 2.0 ** -11, 3.0], [0.5, 1.5, 2.5, 1.0, -0.00146484375]))
        # halfway between 1 + 2^-10 and 1 + 2^-9: goes up to the even 1 + 2^-9
        add("step_tie_up", _fill([-9 * 2.0 ** -11, 3.0], [0.5, 1.5, 2.5, 1.0, 2.0]))

    # subnormal steps: elements m * 2^-24
    sub = 2.0 ** -24
    # step 4 * 2^-24 exactly; odd multiples of 2 * 2^-24 are exact ties
    add("sub_step_exact", _fill([0.0, top * 4 * sub], [2 * k * sub for k in range(2 * top + 1)]))
    add("sub_step_round", _fill([0.0, 7 * sub], [m * sub for m in range(8)]))
    add("sub_step_neg", _fill([-40 * sub, -3 * sub], [-m * sub for m in range(3, 41, 3)]))
    # steps that round to zero: range 2^-24 (B <= 8: range / top < 2^-25
    # for top >= 3), codes all 0 although the group is not constant
    add("zero_step_a", _fill([0.0, sub], [0.0, sub]))
    add("zero_step_b", _fill([2.0 ** -14, 2.0 ** -14 + sub], [2.0 ** -14, 2.0 ** -14 + sub]))

    # zero minima with both signs of zero: the zero point is the first
    # minimal element, so its sign is that of the first zero in index order
    # (the tilers rotate groups, so both orders occur)
    add("zeros_neg_first", _fill([-0.0, 0.0, 1.0, 2.0], [0.5, 1.5, 0.0, -0.0, 3.0]))
    add("zeros_pos_first", _fill([0.0, -0.0, 3.0], [-0.0, 1.0, 0.0, 2.5]))
    add("all_zeros_mixed", _fill([-0.0, 0.0], [0.0, -0.0]))

    # large magnitudes, both signs
    big = np.round(rng.uniform(-60000, 60000, G - 2))
    add("large", [-60000.0, 60000.0] + list(np.float16(big).astype(np.float64)))
    # ordinary draws, and one outlier-scaled draw
    for i in range(3):
        add(f"normal_{i}", np.float16(rng.standard_normal(G)).astype(np.float64))
    add("outlier_x50", np.float16(50 * rng.standard_normal(G)).astype(np.float64))

    if np.dtype(dtype) == np.float32:
        # fp32 inputs: the minimum is not a binary16 value (z16 = RNE16(min)),
        # and elements sit a few fp32 ulps either side of the ties measured
        # from the stored zero and step
        tiny = 2.0 ** -30  # rounds to binary16 0
        vals = [tiny, float(top)]
        k = 0
        while len(vals) < G:
            t = np.float32((k % top) + 0.5)
            for m in (1, 2):
                up, dn = t, t
                for _ in range(m):
                    up = np.nextafter(up, np.float32(np.inf))
                    dn = np.nextafter(dn, np.float32(-np.inf))
                vals += [float(up), float(dn)]
            vals.append(float(t))
            k += 1
        add("f32_near_ties", vals[:G])
        add("f32_offset_min", _fill([1.0 + 2.0 ** -20, 4.0 + 2.0 ** -20],
                                    [1.5 + 2.0 ** -20, 2.5 + 2.0 ** -21, 3.0]))
        add("f32_const_fp16", [1.25] * G)
    return names, np.stack(groups)


def tile_keys(groups, nb, hkv, T, D, seed=0):
    """Keys [nb][hkv][T][D]: full groups of 32 tokens hold one edge group per
    channel (rotated by a channel-dependent amount so the special elements
    land on different tokens); tokens of an unfilled last group are copied
    from the group list as well."""
    N = len(groups)
    k = np.empty((nb, hkv, T, D), dtype=groups.dtype)
    for b in range(nb):
        for h in range(hkv):
            for c in range(D):
                for g in range((T + G - 1) // G):
                    e = (g * D + c + 7 * h + 13 * b + seed) % N
                    r = (3 * c + g + seed) % G
                    col = np.roll(groups[e], r)
                    cnt = min(G, T - g * G)
                    k[b, h, g * G:g * G + cnt, c] = col[:cnt]
    return k


def tile_values(groups, nb, hkv, T, D, seed=0):
    """Values [nb][hkv][T][D]: each token's channel group cg holds one edge
    group (rotated by a token-dependent amount)."""
    N = len(groups)
    ncg = D // G
    v = np.empty((nb, hkv, T, D), dtype=groups.dtype)
    for b in range(nb):
        for h in range(hkv):
            for t in range(T):
                for cg in range(ncg):
                    e = (t * ncg + cg + 5 * h + 11 * b + 3 * seed) % N
                    v[b, h, t, cg * G:(cg + 1) * G] = np.roll(groups[e], (t + cg + seed) % G)
    return v
