// kvq_kernels.hip -- gfx950 kernels: key/value quantize-and-pack, key-tail
// append and flush, decode attention over the quantized cache, split combine.
//
// Method (web pages): uniform asymmetric integer codes per group, zero point
// = group minimum, step = range/(2^B-1), nearest step ("Your KV Cache Doesn't
// Have a Bit Problem...", section "What Quantization Error Is Actually Made
// Of"); keys grouped per channel over G tokens, values per token over G
// channels (same page, "Keys: The Outliers Live in Fixed Channels", "Values:
// Where the Intuition Breaks"); unfilled key groups wait in a full-precision
// tail ("The Systems Tax, and Why It Is Not a Detail"); rotary embedding
// applied to keys after dequantization ("Rotary Embeddings Complicate the
// Keys").
#include "kvq_codec.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>

namespace kvqi {
namespace {

constexpr int G = kGroup;

// ------------------------------------------------------------- binary16 --

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return __half2float(__ushort_as_half((unsigned short)h));
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__half>(__half x) { return __half2float(x); }

// Quantize one group of G values held by one thread and pack it LSB-first.
template <int BITS>
__device__ __forceinline__ uint32_t quantize_pack(const float (&x)[G], uint32_t (&w)[G * BITS / 32])
{
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < G; ++j) {
        mn = fminf(mn, x[j]);
        mx = fmaxf(mx, x[j]);
    }
    const GroupParams gp = group_params(mn, mx, BITS);
#pragma unroll
    for (int i = 0; i < G * BITS / 32; ++i)
        w[i] = 0u;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t c = code_of((double)x[j], gp, (1 << BITS) - 1);
        w[(j * BITS) / 32] |= c << ((j * BITS) % 32);
    }
    return gp.meta;
}

// ------------------------------------------------------- prefill kernels --

// One thread per (sequence*head, key group, channel): walks the group's G
// tokens down the channel, so the per-channel statistics need no cross-lane
// reduction; consecutive threads read consecutive channels of a token row.
template <typename T, int BITS>
__global__ __launch_bounds__(256) void quant_keys_kernel(Planes p, const T* __restrict__ k,
                                                         int n_tokens, int ngroups)
{
    constexpr int WK = G * BITS / 32;
    const int D = p.D;
    const int gpb = blockDim.x / D;
    const int c = threadIdx.x % D;
    const int g = blockIdx.x * gpb + threadIdx.x / D;
    const size_t bh = blockIdx.y;
    if (g >= ngroups)
        return;
    const T* src = k + (bh * (size_t)n_tokens + (size_t)g * G) * D + c;
    float x[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        x[j] = to_f32(src[(size_t)j * D]);
    uint32_t w[WK];
    const uint32_t meta = quantize_pack<BITS>(x, w);
    const size_t gc = (bh * p.gcap + g) * D + c;
    uint32_t* dst = p.k_codes + gc * WK;
#pragma unroll
    for (int i = 0; i < WK; ++i)
        dst[i] = w[i];
    p.k_meta[gc] = meta;
}

// Copy the last n_tokens mod G keys of each sequence/head into the tail.
template <typename T>
__global__ void copy_tail_kernel(Planes p, const T* __restrict__ k, int n_tokens, int tq,
                                 size_t total)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int D = p.D;
    const int rem = n_tokens - tq;
    const int c = idx % D;
    const int j = (idx / D) % rem;
    const size_t bh = idx / ((size_t)D * rem);
    T* tail = reinterpret_cast<T*>(p.k_tail);
    tail[(bh * G + j) * D + c] = k[(bh * n_tokens + tq + j) * D + c];
}

// One thread per (sequence*head, token, channel group): the group is G
// consecutive channels of one token row (64 contiguous bytes at fp16).
// Input tokens [0, n_src) go to cache slots [t_dst0, t_dst0 + n_src).
template <typename T, int BITS>
__global__ __launch_bounds__(256) void quant_values_kernel(Planes p, const T* __restrict__ v,
                                                           int n_src, int t_dst0, size_t total)
{
    constexpr int WV = G * BITS / 32;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int D = p.D;
    const int ncg = D / G;
    const int cg = idx % ncg;
    const size_t r = idx / ncg;
    const int t = r % n_src;
    const size_t bh = r / n_src;
    const T* src = v + (bh * n_src + t) * D + (size_t)cg * G;
    float x[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        x[j] = to_f32(src[j]);
    uint32_t w[WV];
    const uint32_t meta = quantize_pack<BITS>(x, w);
    const size_t tc = (bh * p.tcap + t_dst0 + t) * ncg + cg;
    uint32_t* dst = p.v_codes + tc * WV;
#pragma unroll
    for (int i = 0; i < WV; ++i)
        dst[i] = w[i];
    p.v_meta[tc] = meta;
}

// Append one key per sequence/head into tail slot n mod G; when that slot is
// the last one, quantize the full tail as key group n/G.  One thread per
// channel: every tail element a thread reads was written by the same
// thread's channel (this launch) or by an earlier launch.
template <typename T, int BITS>
__global__ void append_keys_kernel(Planes p, const T* __restrict__ k, int n)
{
    constexpr int WK = G * BITS / 32;
    const int D = p.D;
    const int c = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (c >= D)
        return;
    T* tail = reinterpret_cast<T*>(p.k_tail);
    const int slot = n % G;
    const T val = k[bh * D + c];
    tail[(bh * G + slot) * D + c] = val;
    if (slot != G - 1)
        return;
    float x[G];
#pragma unroll
    for (int j = 0; j < G - 1; ++j)
        x[j] = to_f32(tail[(bh * G + j) * D + c]);
    x[G - 1] = to_f32(val);
    uint32_t w[WK];
    const uint32_t meta = quantize_pack<BITS>(x, w);
    const size_t gc = (bh * p.gcap + n / G) * D + c;
    uint32_t* dst = p.k_codes + gc * WK;
#pragma unroll
    for (int i = 0; i < WK; ++i)
        dst[i] = w[i];
    p.k_meta[gc] = meta;
}

// ------------------------------------------------------ decode attention --

__device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

constexpr float kLog2e = 1.4426950408889634f;

// Reference-structured decode attention (one block per (split, sequence*KV
// head)).  Each block walks its token units (a unit = one key group of G
// tokens, or the tail), computes the scores of every query head that reads
// this KV head, keeps an online softmax (running max m and sum l, base 2),
// accumulates sum p*vhat, and writes (o[D], m, l) to its partial slot.
template <int D, int KB, int VB, typename T>
__global__ __launch_bounds__(256) void attend_ref_kernel(Planes p, const T* __restrict__ q, int n,
                                                         int splits)
{
    constexpr int NP = D / 2;
    constexpr int WK = G * KB / 32, WV = G * VB / 32, NCG = D / G;
    constexpr int PARTS = 256 / G;          // threads per token in the score pass
    constexpr int PPP = NP / PARTS;         // pairs per thread
    constexpr int MAXQ = 8;
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / p.hkv, kvh = bh % p.hkv;
    const int qpk = p.hq / p.hkv;
    const int ngq = n / G;
    const int tq = ngq * G;
    const bool has_tail = n > tq;
    const int units = ngq + (has_tail ? 1 : 0);
    const int u0 = (int)((long long)split * units / splits);
    const int u1 = (int)((long long)(split + 1) * units / splits);

    __shared__ float2 sQ[MAXQ][NP];
    __shared__ float sP[MAXQ][G];
    __shared__ float sAlpha[MAXQ];

    // conj(rotated query) * log2(e)/sqrt(D)
    {
        const int pos = n - 1;
        const float scale = kLog2e * rsqrtf((float)D);
        for (int idx = tid; idx < qpk * NP; idx += blockDim.x) {
            const int hh = idx / NP, i = idx % NP;
            const float2 rot = cmul(p.rope_group[(size_t)(pos / G) * NP + i],
                                    p.rope_offset[(pos % G) * NP + i]);
            const T* qp = q + ((size_t)(b * p.hq + kvh * qpk + hh)) * D + 2 * i;
            const float2 qq = cmul(make_float2(to_f32(qp[0]), to_f32(qp[1])), rot);
            sQ[hh][i] = make_float2(qq.x * scale, -qq.y * scale);
        }
    }
    __syncthreads();

    float m_run[MAXQ], l_run[MAXQ];
    for (int hh = 0; hh < MAXQ; ++hh) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.f;
    }
    constexpr int MAXCOMBO = MAXQ * D / 256;
    float o[MAXCOMBO];
    for (int r = 0; r < MAXCOMBO; ++r)
        o[r] = 0.f;

    const T* tail = reinterpret_cast<const T*>(p.k_tail) + (size_t)bh * G * D;
    for (int u = u0; u < u1; ++u) {
        const bool tail_unit = (u == ngq);
        const int cnt = tail_unit ? n - tq : G;
        const int t0 = u * G;
        // ---- scores: thread (j, part)
        const int j = tid / PARTS, part = tid % PARTS;
        float sc[MAXQ];
        for (int hh = 0; hh < MAXQ; ++hh)
            sc[hh] = 0.f;
        if (j < cnt) {
            for (int ii = 0; ii < PPP; ++ii) {
                const int i = part * PPP + ii;
                float x, y;
                if (tail_unit) {
                    x = to_f32(tail[(size_t)j * D + 2 * i]);
                    y = to_f32(tail[(size_t)j * D + 2 * i + 1]);
                } else {
                    const size_t gc = ((size_t)bh * p.gcap + u) * D + 2 * i;
                    const int bit = j * KB;
                    const uint32_t c0 = (p.k_codes[gc * WK + bit / 32] >> (bit % 32)) & ((1u << KB) - 1u);
                    const uint32_t c1 = (p.k_codes[(gc + 1) * WK + bit / 32] >> (bit % 32)) & ((1u << KB) - 1u);
                    const uint32_t m0 = p.k_meta[gc], m1 = p.k_meta[gc + 1];
                    x = half_bits_to_float(m0 >> 16) + half_bits_to_float(m0 & 0xffffu) * (float)c0;
                    y = half_bits_to_float(m1 >> 16) + half_bits_to_float(m1 & 0xffffu) * (float)c1;
                }
                const float2 rot = cmul(p.rope_group[(size_t)u * NP + i], p.rope_offset[j * NP + i]);
                const float2 kr = cmul(make_float2(x, y), rot);
                for (int hh = 0; hh < qpk; ++hh) {
                    const float2 qc = sQ[hh][i];
                    sc[hh] += qc.x * kr.x - qc.y * kr.y;  // Re[conj(q') k']
                }
            }
        }
        for (int hh = 0; hh < qpk; ++hh) {
            float s = sc[hh];
            for (int off = 1; off < PARTS; off <<= 1)
                s += __shfl_xor(s, off);
            sc[hh] = s;
        }
        // ---- online softmax: every thread of a head row sees all scores
        __shared__ float sS[MAXQ][G];
        if (part == 0)
            for (int hh = 0; hh < qpk; ++hh)
                sS[hh][j] = (j < cnt) ? sc[hh] : -INFINITY;
        __syncthreads();
        if (tid < qpk) {
            const int hh = tid;
            float mx = m_run[hh];
            for (int jj = 0; jj < cnt; ++jj)
                mx = fmaxf(mx, sS[hh][jj]);
            sAlpha[hh] = exp2f(m_run[hh] - mx);  // 0 on the first unit
            float sum = 0.f;
            for (int jj = 0; jj < G; ++jj) {
                const float pj = (jj < cnt) ? exp2f(sS[hh][jj] - mx) : 0.f;
                sP[hh][jj] = pj;
                sum += pj;
            }
            sS[hh][0] = mx;  // broadcast the new max (scores no longer needed)
            sS[hh][1] = sum;
        }
        __syncthreads();
        for (int hh = 0; hh < qpk; ++hh) {
            l_run[hh] = l_run[hh] * sAlpha[hh] + sS[hh][1];
            m_run[hh] = sS[hh][0];
        }
        // ---- values: thread owns (head, channel) combos
        for (int r = 0; r < MAXCOMBO; ++r) {
            const int combo = tid + r * 256;
            if (combo >= qpk * D)
                break;
            const int hh = combo / D, c = combo % D;
            const int cg = c / G, jc = c % G;
            float acc = o[r] * sAlpha[hh];
            for (int jj = 0; jj < cnt; ++jj) {
                const size_t tc = ((size_t)bh * p.tcap + t0 + jj) * NCG + cg;
                const int bit = jc * VB;
                const uint32_t code = (p.v_codes[tc * WV + bit / 32] >> (bit % 32)) & ((1u << VB) - 1u);
                const uint32_t mt = p.v_meta[tc];
                const float vh = half_bits_to_float(mt >> 16) + half_bits_to_float(mt & 0xffffu) * (float)code;
                acc += sP[hh][jj] * vh;
            }
            o[r] = acc;
        }
        __syncthreads();
    }
    // ---- partials
    for (int r = 0; r < MAXCOMBO; ++r) {
        const int combo = tid + r * 256;
        if (combo >= qpk * D)
            break;
        const int hh = combo / D, c = combo % D;
        const size_t row = (size_t)b * p.hq + kvh * qpk + hh;
        float* dst = p.partials + (row * p.max_splits + split) * (D + 2);
        dst[c] = o[r];
        if (c == 0) {
            dst[D] = m_run[hh];
            dst[D + 1] = l_run[hh];
        }
    }
}

// Merge the split partials of one output row: out = sum_s 2^(m_s-M) o_s /
// sum_s 2^(m_s-M) l_s.
__global__ void combine_kernel(const float* __restrict__ partials, int max_splits, int splits,
                               int D, float* __restrict__ out)
{
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const float* base = partials + row * max_splits * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s)
        M = fmaxf(M, base[s * (D + 2) + D]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float w = exp2f(base[s * (D + 2) + D] - M);
        L += w * base[s * (D + 2) + D + 1];
        if (c < D)
            acc += w * base[s * (D + 2) + c];
    }
    if (c < D)
        out[row * D + c] = acc / L;
}

// ------------------------------------------------------------- dispatch --

template <typename T>
hipError_t quantize_prefill_t(const Planes& p, const T* k, const T* v, int n_tokens,
                              hipStream_t stream)
{
    const int ngroups = n_tokens / G;
    const int tq = ngroups * G;
    const int nbh = p.nb * p.hkv;
    if (ngroups > 0) {
        const int gpb = 256 / p.D;
        dim3 grid((ngroups + gpb - 1) / gpb, nbh);
        switch (p.kbits) {
        case 2: quant_keys_kernel<T, 2><<<grid, gpb * p.D, 0, stream>>>(p, k, n_tokens, ngroups); break;
        case 4: quant_keys_kernel<T, 4><<<grid, gpb * p.D, 0, stream>>>(p, k, n_tokens, ngroups); break;
        case 8: quant_keys_kernel<T, 8><<<grid, gpb * p.D, 0, stream>>>(p, k, n_tokens, ngroups); break;
        }
    }
    if (n_tokens > tq) {
        const size_t total = (size_t)nbh * (n_tokens - tq) * p.D;
        copy_tail_kernel<T><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(p, k, n_tokens, tq, total);
    }
    const size_t vg = (size_t)nbh * n_tokens * (p.D / G);
    const unsigned vblocks = (unsigned)((vg + 255) / 256);
    switch (p.vbits) {
    case 2: quant_values_kernel<T, 2><<<vblocks, 256, 0, stream>>>(p, v, n_tokens, 0, vg); break;
    case 4: quant_values_kernel<T, 4><<<vblocks, 256, 0, stream>>>(p, v, n_tokens, 0, vg); break;
    case 8: quant_values_kernel<T, 8><<<vblocks, 256, 0, stream>>>(p, v, n_tokens, 0, vg); break;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t append_t(const Planes& p, const T* k, const T* v, int n, hipStream_t stream)
{
    const int nbh = p.nb * p.hkv;
    switch (p.kbits) {
    case 2: append_keys_kernel<T, 2><<<nbh, p.D, 0, stream>>>(p, k, n); break;
    case 4: append_keys_kernel<T, 4><<<nbh, p.D, 0, stream>>>(p, k, n); break;
    case 8: append_keys_kernel<T, 8><<<nbh, p.D, 0, stream>>>(p, k, n); break;
    }
    const size_t vg = (size_t)nbh * (p.D / G);
    const unsigned vblocks = (unsigned)((vg + 255) / 256);
    switch (p.vbits) {
    case 2: quant_values_kernel<T, 2><<<vblocks, 256, 0, stream>>>(p, v, 1, n, vg); break;
    case 4: quant_values_kernel<T, 4><<<vblocks, 256, 0, stream>>>(p, v, 1, n, vg); break;
    case 8: quant_values_kernel<T, 8><<<vblocks, 256, 0, stream>>>(p, v, 1, n, vg); break;
    }
    return hipGetLastError();
}

template <int D, int KB, int VB, typename T>
void attend_launch(const Planes& p, const void* q, int n, int splits, hipStream_t stream)
{
    dim3 grid(splits, p.nb * p.hkv);
    attend_ref_kernel<D, KB, VB, T><<<grid, 256, 0, stream>>>(p, static_cast<const T*>(q), n, splits);
}

template <int D, int KB, typename T>
void attend_vb(const Planes& p, const void* q, int n, int splits, hipStream_t s)
{
    switch (p.vbits) {
    case 2: attend_launch<D, KB, 2, T>(p, q, n, splits, s); break;
    case 4: attend_launch<D, KB, 4, T>(p, q, n, splits, s); break;
    case 8: attend_launch<D, KB, 8, T>(p, q, n, splits, s); break;
    }
}

template <int D, typename T>
void attend_kb(const Planes& p, const void* q, int n, int splits, hipStream_t s)
{
    switch (p.kbits) {
    case 2: attend_vb<D, 2, T>(p, q, n, splits, s); break;
    case 4: attend_vb<D, 4, T>(p, q, n, splits, s); break;
    case 8: attend_vb<D, 8, T>(p, q, n, splits, s); break;
    }
}

}  // namespace

hipError_t launch_quantize_prefill(const Planes& p, const void* k, const void* v, int n_tokens,
                                   hipStream_t stream)
{
    if (p.dtype == 0)
        return quantize_prefill_t<__half>(p, static_cast<const __half*>(k),
                                          static_cast<const __half*>(v), n_tokens, stream);
    return quantize_prefill_t<float>(p, static_cast<const float*>(k), static_cast<const float*>(v),
                                     n_tokens, stream);
}

hipError_t launch_append(const Planes& p, const void* k, const void* v, int n, hipStream_t stream)
{
    if (p.dtype == 0)
        return append_t<__half>(p, static_cast<const __half*>(k), static_cast<const __half*>(v), n,
                                stream);
    return append_t<float>(p, static_cast<const float*>(k), static_cast<const float*>(v), n, stream);
}

hipError_t launch_attend(const Planes& p, const void* q, float* out, int n, int splits,
                         hipStream_t stream)
{
    if (p.D == 64) {
        if (p.dtype == 0) attend_kb<64, __half>(p, q, n, splits, stream);
        else attend_kb<64, float>(p, q, n, splits, stream);
    } else {
        if (p.dtype == 0) attend_kb<128, __half>(p, q, n, splits, stream);
        else attend_kb<128, float>(p, q, n, splits, stream);
    }
    combine_kernel<<<p.nb * p.hq, p.D, 0, stream>>>(p.partials, p.max_splits, splits, p.D, out);
    return hipGetLastError();
}

}  // namespace kvqi
