// Host build of the GPU library's exact codec helpers (kvq_codec.h), exposed
// through a C ABI so a CPU test can compare them with the oracle.
#include "kvq_codec.h"

extern "C" {
uint32_t shim_double_to_half(double x) { return kvqi::double_to_half_bits(x); }
double shim_half_to_double(uint32_t h) { return kvqi::half_bits_to_double(h); }
// Quantize one group of n floats exactly as the kernels do; returns the meta
// word and writes the codes.
uint32_t shim_quant_group(const float* x, int n, int bits, uint8_t* codes)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    const kvqi::GroupParams g = kvqi::group_params(mn, mx, bits);
    for (int i = 0; i < n; ++i)
        codes[i] = (uint8_t)kvqi::code_of((double)x[i], g, (1 << bits) - 1);
    return g.meta;
}
}
