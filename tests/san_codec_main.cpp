// Driver for the GPU library's group codec (kvq_codec.h) built for the CPU
// under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py): random, constant, tie and tiny-range groups
// through the fp32-input quantizer and the binary16 pair codecs, every code
// checked against the exact per-element code (code_of) of the same group
// parameters.  Exit status 0 and no sanitizer report is the pass.
//
// Test infrastructure only.
#include "kvq_codec.h"

#include <cstdio>
#include <cstring>
#include <random>

static int g_fail = 0;

template <int BITS>
static uint32_t code_in(const uint32_t (&w)[BITS], int j)
{
    return (w[(j * BITS) / 32] >> ((j * BITS) % 32)) & ((1u << BITS) - 1u);
}

static uint16_t to_half(double x) { return (uint16_t)kvqi::double_to_half_bits(x); }

template <int BITS>
static void check_group(const uint16_t (&h)[32])
{
    constexpr int TOP = (1 << BITS) - 1;
    float x[32];
    uint32_t d[16], two[32];
    for (int j = 0; j < 32; ++j)
        x[j] = (float)kvqi::half_bits_to_double(h[j]);
    for (int k = 0; k < 16; ++k)
        d[k] = h[2 * k] | ((uint32_t)h[2 * k + 1] << 16);
    for (int j = 0; j < 32; ++j)  // group 0 in the low halves, its reverse in the high
        two[j] = h[j] | ((uint32_t)h[31 - j] << 16);
    float xr[32];
    for (int j = 0; j < 32; ++j)
        xr[j] = x[31 - j];
    uint32_t w[BITS], wr[BITS], wp[BITS], w0[BITS], w1[BITS], m0, m1;
    const uint32_t meta = kvqi::quantize_group<BITS>(x, w);
    // the reversed group: the same step, and the same zero point but for the
    // sign of a zero minimum (the first zero in the other order)
    const uint32_t meta_r = kvqi::quantize_group<BITS>(xr, wr);
    const uint32_t mp = kvqi::quantize_group_pairs<BITS>(d, wp);
    kvqi::quantize_group_two<BITS>(two, w0, w1, m0, m1);
    if (mp != meta || m0 != meta || m1 != meta_r || (meta ^ meta_r) & ~0x80000000u) {
        ++g_fail;
        if (g_fail < 5)
            std::fprintf(stderr, "B=%d meta %08x pairs %08x two %08x %08x\n", BITS, meta, mp, m0,
                         m1);
    }
    // exact reference codes from the group's binary16 parameters
    kvqi::GroupParams g;
    g.z = kvqi::half_bits_to_double(meta >> 16);
    g.s = kvqi::half_bits_to_double(meta & 0xffffu);
    g.rinv = g.s != 0.0 ? 1.0 / g.s : 0.0;
    for (int j = 0; j < 32; ++j) {
        const uint32_t want = kvqi::code_of((double)x[j], g, TOP);
        if (code_in(w, j) != want || code_in(wp, j) != want || code_in(w0, j) != want ||
            code_in(w1, 31 - j) != want || code_in(wr, 31 - j) != want) {
            ++g_fail;
            if (g_fail < 5)
                std::fprintf(stderr, "B=%d element %d: code mismatch\n", BITS, j);
        }
    }
}

template <int BITS>
static void run(std::mt19937_64& rng)
{
    constexpr int TOP = (1 << BITS) - 1;
    std::normal_distribution<double> normal(0.0, 1.0);
    std::uniform_int_distribution<int> pick(0, TOP - 1);
    uint16_t h[32];
    for (int it = 0; it < 3000; ++it) {
        const int kind = it % 6;
        const double scale = std::pow(10.0, (it % 9) - 4);
        for (int j = 0; j < 32; ++j) {
            double v;
            switch (kind) {
            case 0: v = scale * normal(rng); break;
            case 1: v = 1.25; break;                                 // constant
            case 2: v = (j % 2) * 0x1p-24; break;                    // zero step
            case 3: v = j == 0 ? 0.0 : j == 1 ? TOP : pick(rng) + 0.5;  // exact ties
            case 4: v = (j % 8) * 0x1p-24 * (it % 5 + 1); break;     // subnormal steps
            default: v = scale * 60.0 * normal(rng); break;          // outlier scale
            }
            if (v > 65504.0) v = 65504.0;
            if (v < -65504.0) v = -65504.0;
            h[j] = to_half(v);
        }
        if (it % 7 == 0)
            h[it % 32] = 0x8000;  // a negative zero somewhere
        check_group<BITS>(h);
    }
    // the step function over ranges near binary16 rounding boundaries
    for (int e = -24; e < 15; ++e)
        for (int m = 0; m < 64; ++m) {
            const double b = std::ldexp(1.0 + (2 * m + 1) / 2048.0, e) * TOP;
            for (int k = -2; k <= 2; ++k) {
                const double r = b + k * 0x1p-24;
                const float ip = (float)std::floor(r), fr = (float)(r - std::floor(r));
                (void)kvqi::half_step_bits<BITS>(-fr, ip);
            }
        }
}

int main()
{
    std::mt19937_64 rng(12345);
    run<2>(rng);
    run<4>(rng);
    run<8>(rng);
    if (g_fail) {
        std::fprintf(stderr, "%d failures\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
