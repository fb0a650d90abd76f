// kvq_codec.h -- exact binary16 conversions and the code of one element,
// usable on the host and the device (the host build lets the CPU tests run
// this exact code without a GPU).  Part of the GPU library.
//
// Quantizer (web page "Your KV Cache Doesn't Have a Bit Problem...", section
// "What Quantization Error Is Actually Made Of"): zero point = group minimum,
// step = range / (2^B - 1), each element rounded to the nearest step.
// Readings: binary16 zero and step rounded once to nearest-even, exact ties
// to the even code, codes clamped to [0, 2^B - 1], zero step -> code 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace kvqi {

#define KVQ_HD __host__ __device__ __forceinline__

// ------------------------------------------------------------- binary16 --

// binary16 bits -> double (exact), from the format's definition.
KVQ_HD double half_bits_to_double(uint32_t h)
{
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    double v;
    if (e == 0)
        v = (double)m * 5.9604644775390625e-08;  // m * 2^-24
    else
        v = __builtin_bit_cast(double, (((uint64_t)(e + 1008u)) << 52) | ((uint64_t)m << 42));
    return (h & 0x8000u) ? -v : v;
}

// double -> binary16 bits, one rounding to nearest-even, subnormals kept,
// |x| >= 65520 -> infinity.  Works on the double's bit fields.
KVQ_HD uint32_t double_to_half_bits(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7fffffffffffffffull;
    if (a >= 0x40effe0000000000ull)  // 65520.0
        return sign | 0x7c00u;
    const int bexp = (int)(a >> 52);
    if (bexp == 0)
        return sign;  // zero or a double subnormal: far below 2^-25
    const int exp = bexp - 1023;
    const uint64_t m = (a & 0xfffffffffffffull) | (1ull << 52);
    int sh;
    uint32_t hi;
    if (exp >= -14) {
        sh = 42;  // keep 11 significant bits
        hi = (uint32_t)(exp + 15) << 10;
    } else {
        sh = 28 - exp;  // units of 2^-24
        hi = 0;
        if (sh > 63)
            return sign;
    }
    uint64_t r = m >> sh;
    const uint64_t rem = m & ((1ull << sh) - 1ull);
    const uint64_t halfway = 1ull << (sh - 1);
    if (rem > halfway || (rem == halfway && (r & 1ull)))
        r += 1;
    if (exp >= -14)
        return sign | (hi + (uint32_t)r - 1024u);  // r may carry into exponent
    return sign | (uint32_t)r;
}

// ------------------------------------------------------------ quantizer --

struct GroupParams {
    double z, s, rinv;
    float zf, rinvf;  // z exactly, 1/s rounded once to fp32
    uint32_t meta;    // step bits | zero bits << 16
};

// Zero point and step of a group with minimum mn and maximum mx, each
// rounded once to binary16.  mx - mn is exact in fp64 for binary16 and
// ordinary fp32 inputs; the fp64 quotient rounds to the same binary16 as the
// exact quotient (it cannot cross a binary16 rounding boundary).
KVQ_HD GroupParams group_params(float mn, float mx, int bits)
{
    const double dmn = (double)mn, dmx = (double)mx;
    const uint32_t z16 = double_to_half_bits(dmn);
    const uint32_t s16 = double_to_half_bits((dmx - dmn) / (double)((1 << bits) - 1));
    GroupParams g;
    g.z = half_bits_to_double(z16);
    g.s = half_bits_to_double(s16);
    g.rinv = (g.s != 0.0) ? 1.0 / g.s : 0.0;
    g.zf = (float)g.z;
    g.rinvf = (float)g.rinv;
    g.meta = s16 | (z16 << 16);
    return g;
}

// Nearest integer to (x - z)/s, exact ties to even, clamped to [0, top].
// d = x - z is exact; q = d * (1/s) is within 2^-44 of the exact quotient
// (|quotient| <= 256), while an exact quotient that is not a tie lies at
// least 2^-41 from every half-integer, so rint(q) is the exact nearest
// integer except at exact ties, which the exact residual e = d - c*s
// (|e| = s/2) detects.
KVQ_HD uint32_t code_of(double x, const GroupParams& g, int top)
{
    if (g.s == 0.0)
        return 0u;
    const double d = x - g.z;
    double c = rint(d * g.rinv);
    const double e = fma(-c, g.s, d);
    if (2.0 * fabs(e) == g.s && ((long long)c & 1))  // exact tie, c odd: take the even neighbour
        c += (e > 0.0 ? 1.0 : -1.0);
    c = fmin(fmax(c, 0.0), (double)top);
    return (uint32_t)c;
}

// The same code through fp32 where fp32 decides it.  For x and z in binary16
// or fp32, q32 = fl(fl(x - z) * fl(1/s)) carries three roundings, so
// |q32 - q| <= 3.0001 * 2^-24 * |q|; when q32 is farther than
// 2^-21 * (|q32| + 1) from every half-integer, q and q32 have the same
// nearest integer and rint(q32) is the code.  q32 - rint(q32) is exact
// (Sterbenz).  The rare elements inside that band take code_of.
// The exact path for one element, from the group's fp64 parameters.  Kept
// inline: the kernels branch to it rarely, and an out-of-line call gives
// every wave a call frame to set up.
KVQ_HD uint32_t code_of_exact(float x, double z, double s, double rinv, int top)
{
    GroupParams g;
    g.z = z;
    g.s = s;
    g.rinv = rinv;
    return code_of((double)x, g, top);
}

KVQ_HD uint32_t code_of_fast(float x, const GroupParams& g, int top)
{
    const float q = (x - g.zf) * g.rinvf;
    const float c = rintf(q);
    const float t = fabsf(q - c);
    if (fabsf(t - 0.5f) <= 0x1p-21f * (fabsf(q) + 1.0f))
        return code_of_exact(x, g.z, g.s, g.rinv, top);
    return (uint32_t)fminf(fmaxf(c, 0.0f), (float)top);
}

// Quantize one group of 32 values and pack the codes LSB-first into B words,
// the codes computed in fp32 as in code_of_fast.  A half-integer h changes a
// clamped code only for h in [-0.5, 2^B - 1.5], where the fp32 quotient is
// within 3 * 2^-24 * (2^B + 1) < 2^-21 * (2^B + 1) of the exact one.  For
// B <= 4 the group keeps the largest |q - rint(q)| and is recomputed exactly
// when that reaches 0.5 - 2^-21 * (2^B + 1); for B = 8 a large share of
// groups would, so each element checks its own band (code_of_fast).
template <int BITS>
KVQ_HD uint32_t quantize_group(const float (&x)[32], uint32_t (&w)[BITS])
{
    constexpr int TOP = (1 << BITS) - 1;
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        mn = fminf(mn, x[j]);
        mx = fmaxf(mx, x[j]);
    }
    const GroupParams gp = group_params(mn, mx, BITS);
#pragma unroll
    for (int i = 0; i < BITS; ++i)
        w[i] = 0u;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = code_of_fast(x[j], gp, TOP);
            w[(j * BITS) / 32] |= c << ((j * BITS) % 32);
        }
    } else {
        float tmax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const float q = (x[j] - gp.zf) * gp.rinvf;
            const float c = rintf(q);
            tmax = fmaxf(tmax, fabsf(q - c));
            const uint32_t ci = (uint32_t)fminf(fmaxf(c, 0.0f), (float)TOP);
            w[(j * BITS) / 32] |= ci << ((j * BITS) % 32);
        }
        if (tmax >= 0.5f - 0x1p-21f * (float)(TOP + 2)) {
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                w[i] = 0u;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t c = code_of_exact(x[j], gp.z, gp.s, gp.rinv, TOP);
                w[(j * BITS) / 32] |= c << ((j * BITS) % 32);
            }
        }
    }
    return gp.meta;
}

}  // namespace kvqi
