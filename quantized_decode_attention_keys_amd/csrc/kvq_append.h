// kvq_append.h -- device helpers that append one token to the quantized
// cache: the per-token value codec and the per-channel key tail with its
// group flush.  Used by the append kernel and by the decode-attention kernel
// when it appends the new token itself (one launch per decode step).
//
// Method (web pages): values are quantized per token as soon as they arrive,
// keys wait in a full-precision tail until G of them fill a per-channel group
// ("Your KV Cache Doesn't Have a Bit Problem...", section "The Systems Tax,
// and Why It Is Not a Detail"; grouping from "Keys: The Outliers Live in
// Fixed Channels" and "Values: Where the Intuition Breaks").
#pragma once

#include "kvq_codec.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>

namespace kvqi {
namespace {

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__half>(__half x) { return __half2float(x); }

// Append one token of an operand grouped per token (G channels of one
// token row) at cache slot n: thread c = channel c of the row.  The 32 lanes
// of a channel group find the group's min and max with lane shuffles, each
// codes its own element, and the codes are OR-reduced into 32-bit words
// across the lanes that share a word.  Every lane of the block must call it.
template <typename T, int BITS>
__device__ __forceinline__ void append_token_groups(uint32_t* __restrict__ codes,
                                                    uint32_t* __restrict__ meta, int tcap,
                                                    const T* __restrict__ row, size_t bh, int n,
                                                    int c, int D)
{
    constexpr int CPW = 32 / BITS;  // codes per 32-bit word
    const float x = to_f32(row[c]);
    float mn = x, mx = x;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {  // within the 32-lane group
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    // the zero point is the first minimal element: for a zero minimum the
    // first zero in channel order gives its sign (the condition holds for all
    // 32 lanes of the group or none)
    if (mn == 0.0f) {
        const unsigned long long zb = __ballot(x == 0.0f);
        const int base = (threadIdx.x & 63) & ~31;
        mn = __shfl(x, base + __builtin_ctz((uint32_t)(zb >> base)));
    }
    const GroupParams gp = group_params(mn, mx, BITS);
    const int j = c % kGroup;
    uint32_t bits = code_of_fast(x, gp, (1 << BITS) - 1) << ((j * BITS) % 32);
#pragma unroll
    for (int off = CPW / 2; off >= 1; off >>= 1)
        bits |= __shfl_xor(bits, off);
    const int ncg = D / kGroup, cg = c / kGroup;
    const size_t tc = (bh * tcap + n) * ncg + cg;
    if (j % CPW == 0)
        codes[tc * (kGroup * BITS / 32) + (j * BITS) / 32] = bits;
    if (j == 0)
        meta[tc] = gp.meta;
}

// Append one token of an operand grouped per channel (one channel over G
// tokens): thread c writes channel c into tail slot n mod G and, when that
// slot is the group's last, quantizes the G tail elements of channel c as
// group n/G.  Every tail element a thread reads was written by the same
// thread (this launch) or by an earlier launch.
template <typename T, int BITS>
__device__ __forceinline__ void append_channel_groups(uint32_t* __restrict__ codes,
                                                      uint32_t* __restrict__ meta, int gcap,
                                                      T* __restrict__ tail, T val, size_t bh,
                                                      int n, int c, int D)
{
    constexpr int W = kGroup * BITS / 32;
    const int slot = n % kGroup;
    tail[slot * D + c] = val;
    if (slot != kGroup - 1)
        return;
    float x[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup - 1; ++j)
        x[j] = to_f32(tail[j * D + c]);
    x[kGroup - 1] = to_f32(val);
    uint32_t w[W];
    const uint32_t m = quantize_group<BITS>(x, w);
    const size_t gc = (bh * gcap + n / kGroup) * D + c;
#pragma unroll
    for (int i = 0; i < W; ++i)
        codes[gc * W + i] = w[i];
    meta[gc] = m;
}

}  // namespace
}  // namespace kvqi
