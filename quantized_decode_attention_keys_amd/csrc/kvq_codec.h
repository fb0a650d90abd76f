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
    // fabs: a group of zeros of both signs may give -0 here; the step is +0
    const uint32_t s16 = double_to_half_bits(fabs(dmx - dmn) / (double)((1 << bits) - 1));
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
    // the zero point is the first minimal element: for a zero minimum, the
    // first zero in index order gives its sign
    if (mn == 0.0f) {
        for (int j = 0; j < 32; ++j)
            if (x[j] == 0.0f) {
                mn = x[j];
                break;
            }
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

// ------------------------------------------------ binary16 group codec --
//
// The same quantizer for binary16 inputs held as packed pairs (two values
// per 32-bit word), with less arithmetic per element than the fp32-input
// path above:
//   - minimum and maximum over packed pairs (exact for binary16); the zero
//     point is the minimum itself (no rounding), and with a zero minimum
//     the first zero in index order gives its sign, as the minimum is the
//     first minimal element;
//   - the step from an fp64 product and a round-to-odd through fp32
//     (half_step_bits), without a division;
//   - each quotient as one fused multiply-add of the binary16 operand,
//     q = x * r + (-z * r) with r ~ 1/step, and codes packed four, two or
//     one to a byte from their float values;
//   - the fast codes are kept when every |q - rint(q)| stays below
//     1/2 - band, band a per-group bound eight times the error of q
//     (GroupH), and recomputed exactly (code_of_exact) otherwise: for
//     B <= 4 per group, for B = 8 per element.
// A normal binary16 step needs no clamp: every exact quotient lies in
// [0, (2^B - 1)(1 + 2^-11)], below 2^B - 1/2; a zero or subnormal step
// (rounded by up to half of itself) sends the group down the exact path.

#if defined(__HIP_DEVICE_COMPILE__)
typedef _Float16 kvq_h2 __attribute__((ext_vector_type(2)));
#endif

// Low and high binary16 values of a packed word, as floats (exact).
KVQ_HD float h16_lo(uint32_t d)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return (float)__builtin_bit_cast(kvq_h2, d).x;
#else
    return (float)half_bits_to_double(d & 0xffffu);
#endif
}
KVQ_HD float h16_hi(uint32_t d)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return (float)__builtin_bit_cast(kvq_h2, d).y;
#else
    return (float)half_bits_to_double(d >> 16);
#endif
}

// Lane-wise minimum and maximum of N packed pairs of finite binary16 values
// (low halves together, high halves together), as packed words.  Which
// zero comes back for a zero extreme is left open; callers fix the zero
// point's sign.
template <int N>
KVQ_HD void minmax_pairs(const uint32_t (&d)[N], uint32_t& mn, uint32_t& mx)
{
#if defined(__HIP_DEVICE_COMPILE__)
    // IEEE 754-2019 minimum/maximum: no canonicalizing of the loaded
    // operands, three operands per instruction
    kvq_h2 a = __builtin_bit_cast(kvq_h2, d[0]), b = a;
#pragma unroll
    for (int k = 1; k < N; ++k) {
        const kvq_h2 v = __builtin_bit_cast(kvq_h2, d[k]);
        a = __builtin_elementwise_minimum(a, v);
        b = __builtin_elementwise_maximum(b, v);
    }
    mn = __builtin_bit_cast(uint32_t, a);
    mx = __builtin_bit_cast(uint32_t, b);
#else
    uint32_t lo_mn = d[0] & 0xffffu, lo_mx = lo_mn, hi_mn = d[0] >> 16, hi_mx = hi_mn;
    for (int k = 1; k < N; ++k) {
        const uint32_t lo = d[k] & 0xffffu, hi = d[k] >> 16;
        if (half_bits_to_double(lo) < half_bits_to_double(lo_mn)) lo_mn = lo;
        if (half_bits_to_double(lo) > half_bits_to_double(lo_mx)) lo_mx = lo;
        if (half_bits_to_double(hi) < half_bits_to_double(hi_mn)) hi_mn = hi;
        if (half_bits_to_double(hi) > half_bits_to_double(hi_mx)) hi_mx = hi;
    }
    mn = lo_mn | (hi_mn << 16);
    mx = lo_mx | (hi_mx << 16);
#endif
}

// Bits of the zero point of a group whose minimum is mn (bits mn_bits):
// with a zero minimum, the first zero in index order (bits_at(j)).
template <typename Bits>
KVQ_HD uint32_t zero_bits(float mn, uint32_t mn_bits, Bits bits_at)
{
    if (__builtin_expect(mn != 0.0f, 1))
        return mn_bits;
    // rare: a loop, so that the compares stay inside this branch
#pragma clang loop unroll(disable)
    for (int j = 0; j < 32; ++j) {
        const uint32_t b = bits_at(j);
        if ((b & 0x7fffu) == 0u)
            return b;
    }
    return 0u;
}

// float -> binary16 bits, one rounding to nearest-even (subnormals kept).
KVQ_HD uint32_t float_to_half_rne(float f)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(unsigned short, (_Float16)f);
#else
    return double_to_half_bits((double)f);
#endif
}

// Step bits of a group of binary16 values with minimum mn and maximum mx:
// the binary16 nearest (ties to even) to (mx - mn) / (2^B - 1).
//   d = |mx - mn| is exact in fp64 (a multiple of 2^-24 below 2^17), and
//   q = fl(d * fl(1/TOP)) is within 2^-51.9 |q| of the exact quotient, less
//   than 2^-36.  A binary16 rounding boundary m (a multiple of 2^-25) that
//   the exact quotient misses is at least 2^-25 / TOP >= 2^-33 away from it
//   (d - TOP m is a non-zero multiple of 2^-25), so q rounds like the exact
//   quotient; one that it meets comes out of the product exactly (fl(1/TOP)
//   is within 2^-54 of 1/TOP for TOP = 3, 15, 255).
//   q is rounded to odd at fp32 precision (24 >= 11 + 2 bits), after which
//   one rounding to nearest-even binary16 equals that of q itself.
template <int BITS>
KVQ_HD uint32_t half_step_bits(float mn, float mx)
{
    constexpr double kInvTop = 1.0 / (double)((1 << BITS) - 1);
    const double q = fabs((double)mx - (double)mn) * kInvTop;
    const float f = (float)q;  // nearest
    const double back = (double)f;
    uint32_t fb = __builtin_bit_cast(uint32_t, f);
    if (back > q)
        fb -= 1u;  // toward zero (q >= 0)
    if (back != q)
        fb |= 1u;  // sticky: inexact results end odd
    return float_to_half_rne(__builtin_bit_cast(float, fb));
}

// ~1/s for a step s >= 2^-24: within one fp32 ulp.
KVQ_HD float approx_rcp(float s)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_rcpf(s);
#else
    return 1.0f / s;
#endif
}

// Byte i of acc replaced by the integer value of b (an integer in [0, 255]).
KVQ_HD uint32_t put_byte(float b, int i, uint32_t acc)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_cvt_pk_u8_f32(b, (unsigned)i, acc);
#else
    return (acc & ~(0xffu << (8 * i))) | ((uint32_t)b << (8 * i));
#endif
}

struct GroupH {
    float z, s;      // zero point (the minimum), step
    float r, nzr;    // ~1/step (0 for a zero step) and -z * r, each rounded once
    float band;      // bound on |q - exact quotient|, times eight
    uint32_t meta;   // step bits | zero bits << 16
};

// Error of q = fl(x * r + nzr) against Q = (x - z) / s, with
// |r - 1/s| <= 2^-23 / s and nzr = fl(-z r):
//   x r + nzr - Q = (x - z)(r - 1/s) + (nzr + z r),
// so |q - Q| <= 2^-24 (3 |Q| + |z| r) (1 + 2^-20), and with a normal step
// |Q| <= (2^B - 1)(1 + 2^-11) < 2^B; band = 2^-21 (2^B + 1 + |z| r) is
// eight times that bound and more.
template <int BITS>
KVQ_HD GroupH group_params_h(float mn, float mx, uint32_t z16)
{
    constexpr int TOP = (1 << BITS) - 1;
    const uint32_t s16 = half_step_bits<BITS>(mn, mx);
    GroupH g;
    g.z = mn;
    g.s = h16_lo(s16);
    g.r = s16 != 0u ? approx_rcp(g.s) : 0.0f;
    g.nzr = -mn * g.r;
    g.band = 0x1p-21f * ((float)(TOP + 2) + fabsf(mn) * g.r);
    g.meta = s16 | (z16 << 16);
    return g;
}

// Codes of the 32 elements x_at(j) (binary16 values as floats) of a group
// with parameters g and a normal step, packed LSB-first into BITS words
// (element j at bit j * BITS), the bytes built from the codes as floats.
// Returns the largest |q - rint(q)|.
template <int BITS, typename Val>
KVQ_HD float codes_h_fast(Val x_at, const GroupH& g, uint32_t (&w)[BITS])
{
    constexpr int PER_BYTE = 8 / BITS, PER_WORD = 32 / BITS;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
        uint32_t acc = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float b = 0.f;
#pragma unroll
            for (int e = PER_BYTE - 1; e >= 0; --e) {
                const float q = fmaf(x_at(k * PER_WORD + i * PER_BYTE + e), g.r, g.nzr);
                const float c = rintf(q);
                t = fmaxf(t, fabsf(q - c));
                b = e == PER_BYTE - 1 ? c : fmaf(b, (float)(1 << BITS), c);
            }
            acc = put_byte(b, i, acc);
        }
        w[k] = acc;
    }
    return t;
}

// The exact codes of the group (code_of for every element).
template <int BITS, typename Val>
KVQ_HD void codes_h_exact(Val x_at, const GroupH& g, uint32_t (&w)[BITS])
{
    constexpr int TOP = (1 << BITS) - 1;
    const double z = (double)g.z, sd = (double)g.s, rinv = sd != 0.0 ? 1.0 / sd : 0.0;
#pragma unroll
    for (int i = 0; i < BITS; ++i)
        w[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j)
        w[(j * BITS) / 32] |= code_of_exact(x_at(j), z, sd, rinv, TOP) << ((j * BITS) % 32);
}

template <int BITS, typename Val>
KVQ_HD void codes_h(Val x_at, const GroupH& g, uint32_t (&w)[BITS])
{
    constexpr int TOP = (1 << BITS) - 1;
    // a zero or subnormal step (exponent field zero: rare) takes the exact
    // path, so the fast codes need no clamp
    const bool normal_step = (g.meta & 0x7c00u) != 0u;
    if constexpr (BITS == 8) {
        // per element: a group-level test would send a few percent of the
        // groups down the exact path at 8 bits
        const float lim = normal_step ? 0.5f - g.band : -1.0f;
        const double z = (double)g.z, sd = (double)g.s;
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
            uint32_t acc = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = x_at(4 * k + i);
                const float q = fmaf(x, g.r, g.nzr);
                float c = rintf(q);
                if (fabsf(q - c) >= lim)
                    c = (float)code_of_exact(x, z, sd, sd != 0.0 ? 1.0 / sd : 0.0, TOP);
                acc = put_byte(c, i, acc);
            }
            w[k] = acc;
        }
    } else {
        bool exact = true;
        if (normal_step)
            exact = codes_h_fast<BITS>(x_at, g, w) >= 0.5f - g.band;
        if (exact)
            codes_h_exact<BITS>(x_at, g, w);
    }
}

// One group of 32 binary16 values packed as 16 words (element 2k in the low
// half of word k, 2k+1 in the high half): codes into w, returns the meta word.
template <int BITS>
KVQ_HD uint32_t quantize_group_pairs(const uint32_t (&d)[16], uint32_t (&w)[BITS])
{
    uint32_t mn2, mx2;
    minmax_pairs(d, mn2, mx2);
    const float mlo = h16_lo(mn2), mhi = h16_hi(mn2);
    const float mn = fminf(mlo, mhi), mx = fmaxf(h16_lo(mx2), h16_hi(mx2));
    const uint32_t z16 = zero_bits(mn, mlo <= mhi ? (mn2 & 0xffffu) : (mn2 >> 16),
                                   [&](int j) { return (d[j >> 1] >> (16 * (j & 1))) & 0xffffu; });
    const GroupH g = group_params_h<BITS>(mn, mx, z16);
    codes_h<BITS>([&](int j) { return (j & 1) ? h16_hi(d[j >> 1]) : h16_lo(d[j >> 1]); }, g, w);
    return g.meta;
}

// Two groups at once: element j of group 0 in the low half of d[j], of group
// 1 in the high half (two channels of the same 32 tokens).
template <int BITS>
KVQ_HD void quantize_group_two(const uint32_t (&d)[32], uint32_t (&w0)[BITS], uint32_t (&w1)[BITS],
                               uint32_t& meta0, uint32_t& meta1)
{
    uint32_t mn2, mx2;
    minmax_pairs(d, mn2, mx2);
    {
        const float mn = h16_lo(mn2);
        const uint32_t z16 = zero_bits(mn, mn2 & 0xffffu, [&](int j) { return d[j] & 0xffffu; });
        const GroupH g = group_params_h<BITS>(mn, h16_lo(mx2), z16);
        codes_h<BITS>([&](int j) { return h16_lo(d[j]); }, g, w0);
        meta0 = g.meta;
    }
    {
        const float mn = h16_hi(mn2);
        const uint32_t z16 = zero_bits(mn, mn2 >> 16, [&](int j) { return d[j] >> 16; });
        const GroupH g = group_params_h<BITS>(mn, h16_hi(mx2), z16);
        codes_h<BITS>([&](int j) { return h16_hi(d[j]); }, g, w1);
        meta1 = g.meta;
    }
}

}  // namespace kvqi
