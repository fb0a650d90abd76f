// Host build of the GPU library's exact codec helpers (kvq_codec.h), exposed
// through a C ABI so a CPU test can compare them with the oracle.
#include "kvq_codec.h"

extern "C" {
uint32_t shim_double_to_half(double x) { return kvqi::double_to_half_bits(x); }
double shim_half_to_double(uint32_t h) { return kvqi::half_bits_to_double(h); }
// Quantize one group of n = 32 floats with the kernels' group quantizer;
// returns the meta word and writes the unpacked codes.
uint32_t shim_quant_group(const float* x, int n, int bits, uint8_t* codes)
{
    if (n != 32)
        return 0xffffffffu;
    float xs[32];
    for (int i = 0; i < 32; ++i)
        xs[i] = x[i];
    uint32_t w[8] = {0}, meta = 0;
    switch (bits) {
    case 2: meta = kvqi::quantize_group<2>(xs, *reinterpret_cast<uint32_t(*)[2]>(w)); break;
    case 4: meta = kvqi::quantize_group<4>(xs, *reinterpret_cast<uint32_t(*)[4]>(w)); break;
    case 8: meta = kvqi::quantize_group<8>(xs, *reinterpret_cast<uint32_t(*)[8]>(w)); break;
    }
    for (int i = 0; i < n; ++i)
        codes[i] = (uint8_t)((w[(i * bits) / 32] >> ((i * bits) % 32)) & ((1u << bits) - 1u));
    return meta;
}
// The exact fp64 code alone, and the number of elements of a group that the
// fp32 path hands to it.
uint32_t shim_quant_group_exact(const float* x, int n, int bits, uint8_t* codes)
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
// The binary16 codec's step: the binary16 nearest to (mx - mn) / (2^bits - 1)
// for binary16 mn <= mx.
uint32_t shim_half_step(float mn, float mx, int bits)
{
    switch (bits) {
    case 2: return kvqi::half_step_bits<2>(mn, mx);
    case 4: return kvqi::half_step_bits<4>(mn, mx);
    case 8: return kvqi::half_step_bits<8>(mn, mx);
    }
    return 0xffffffffu;
}
// The binary16 codec: one group of 32 values given as 16 packed words, and
// two groups given as 32 words (group 0 in the low halves).
uint32_t shim_quant_pairs(const uint32_t* d, int bits, uint8_t* codes)
{
    uint32_t dd[16];
    for (int i = 0; i < 16; ++i)
        dd[i] = d[i];
    uint32_t w[8] = {0}, meta = 0;
    switch (bits) {
    case 2: meta = kvqi::quantize_group_pairs<2>(dd, *reinterpret_cast<uint32_t(*)[2]>(w)); break;
    case 4: meta = kvqi::quantize_group_pairs<4>(dd, *reinterpret_cast<uint32_t(*)[4]>(w)); break;
    case 8: meta = kvqi::quantize_group_pairs<8>(dd, *reinterpret_cast<uint32_t(*)[8]>(w)); break;
    }
    for (int i = 0; i < 32; ++i)
        codes[i] = (uint8_t)((w[(i * bits) / 32] >> ((i * bits) % 32)) & ((1u << bits) - 1u));
    return meta;
}
void shim_quant_two(const uint32_t* d, int bits, uint8_t* codes0, uint8_t* codes1,
                    uint32_t* metas)
{
    uint32_t dd[32];
    for (int i = 0; i < 32; ++i)
        dd[i] = d[i];
    uint32_t w0[8] = {0}, w1[8] = {0};
    switch (bits) {
    case 2: kvqi::quantize_group_two<2>(dd, *reinterpret_cast<uint32_t(*)[2]>(w0), *reinterpret_cast<uint32_t(*)[2]>(w1), metas[0], metas[1]); break;
    case 4: kvqi::quantize_group_two<4>(dd, *reinterpret_cast<uint32_t(*)[4]>(w0), *reinterpret_cast<uint32_t(*)[4]>(w1), metas[0], metas[1]); break;
    case 8: kvqi::quantize_group_two<8>(dd, *reinterpret_cast<uint32_t(*)[8]>(w0), *reinterpret_cast<uint32_t(*)[8]>(w1), metas[0], metas[1]); break;
    }
    for (int i = 0; i < 32; ++i) {
        codes0[i] = (uint8_t)((w0[(i * bits) / 32] >> ((i * bits) % 32)) & ((1u << bits) - 1u));
        codes1[i] = (uint8_t)((w1[(i * bits) / 32] >> ((i * bits) % 32)) & ((1u << bits) - 1u));
    }
}
int shim_fallbacks(const float* x, int n, int bits)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    const kvqi::GroupParams g = kvqi::group_params(mn, mx, bits);
    int k = 0;
    for (int i = 0; i < n; ++i) {
        const float q = (x[i] - g.zf) * g.rinvf;
        const float t = fabsf(q - rintf(q));
        k += fabsf(t - 0.5f) <= 0x1p-21f * (fabsf(q) + 1.0f);
    }
    return k;
}
}
