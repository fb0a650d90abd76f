// kvq_fp8.hip -- gfx950 kernels for the FP8 (OCP E4M3) cache: encode on
// prefill and append, and decode attention over the bytes.
//
// FP8 is the production default the pages compare against ("Rotate, Then
// Round: The Geometry of KV-Cache Compression", key takeaways: twice the
// capacity of fp16 at small accuracy cost).  Every key and value element is
// one E4M3 byte (bias 7, largest finite 448), rounded to nearest with ties to
// even and saturated at +-448, with no scale factor; keys are stored before
// the rotary embedding, which attention applies after decoding, as in the
// integer cache.
//
// Layout: one D * 32-byte block per (sequence*head, 32-token group) in the
// K_CODES and V_CODES planes (sized for 8-bit codes), made of 16-byte pieces:
// channel c, token j at ((2 (c mod 2) + j div 16) (D/2) + c div 2) 16 + j mod 16.
// The lane that owns channel pair i reads its 64 bytes (both channels, 32
// tokens) as four 16-byte loads at a stride of D * 8 bytes, so each load
// instruction of a wave covers one contiguous (D/2) * 16-byte span; one
// v_cvt_pk_f32_fp8 then decodes two tokens of one channel.  FP8 needs no
// group statistics, so an append writes its byte at once (and clears the
// channel's two pieces when it opens a group, so unwritten bytes decode to 0).
//
// Attention: grid (splits, batch * q_heads), 4 waves; each wave takes whole
// 32-token groups with its own online softmax; it prefetches the next
// group's 64 key bytes per lane while it computes the current one, and loads
// the current values before the scores that they wait behind.  Per (pair,
// token): half a decode, 2 FMAs for Re[P_j (x + i y)] and 4 to advance the
// rotated query P_j = conj(q') e^{i t theta} to the token after next (four
// recurrences per group from table values, at most 8 steps each, no LDS).  The 32 partial scores of a lane are summed across
// the wave by a halving exchange (two lane-swap steps across rows, then DPP
// mirrors inside rows), after which lanes 2j and 2j+1 hold token j.
#include "kvq_attend_kernel.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>

namespace kvqi {
namespace {

template <typename T> __device__ __forceinline__ float lde(const T* p, size_t i);
template <> __device__ __forceinline__ float lde<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float lde<__half>(const __half* p, size_t i)
{
    return __half2float(p[i]);
}

// Nearest E4M3 byte to x, ties to even, |x| >= 448 saturates (x finite).
// Scaling by powers of two is exact in fp32, so rintf rounds the exact value.
__device__ __forceinline__ uint32_t fp8_e4m3(float x)
{
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a < 448.0f))
        return sign | 0x7Eu;
    if (a < 0x1p-6f)  // subnormal steps of 2^-9; code 8 is the smallest normal
        return sign | (uint32_t)rintf(a * 512.0f);
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // a in [2^e, 2^(e+1))
    float qm = rintf(ldexpf(a, 3 - e));                       // 8 .. 16
    if (qm >= 16.0f) {
        qm = 8.0f;
        e += 1;
    }
    return sign | (uint32_t)(((e + 7) << 3) | ((int)qm - 8));
}

// Byte offset of channel c, token j (< 32) inside a group block.
__device__ __forceinline__ size_t fp8_offset(int D, int c, int j)
{
    return ((size_t)(2 * (c % 2) + j / 16) * (D / 2) + c / 2) * 16 + j % 16;
}

// One thread per (sequence*head, group, channel): the 32 tokens of channel c
// of group g (tokens past n_tokens as 0) into its two 16-byte pieces.
template <typename T>
__global__ __launch_bounds__(256) void fp8_prefill_kernel(uint32_t* __restrict__ dst,
                                                          const T* __restrict__ src,
                                                          int n_tokens, int groups, int gcap,
                                                          int D)
{
    const int gpb = blockDim.x / D;
    const int c = threadIdx.x % D;
    const int g = blockIdx.x * gpb + threadIdx.x / D;
    const size_t bh = blockIdx.y;
    if (g >= groups)
        return;
    const T* s = src + (bh * (size_t)n_tokens + (size_t)g * G) * D + c;
    const int cnt = min(G, n_tokens - g * G);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = 4 * k + b;
            if (j < cnt)
                v |= fp8_e4m3(lde(s, (size_t)j * D)) << (8 * b);
        }
        w[k] = v;
    }
    uint8_t* blk = reinterpret_cast<uint8_t*>(dst) + (bh * gcap + g) * (size_t)D * G;
    *reinterpret_cast<uint4*>(blk + fp8_offset(D, c, 0)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(blk + fp8_offset(D, c, 16)) = make_uint4(w[4], w[5], w[6], w[7]);
}

// Append token n: block per sequence*head, thread c = channel c.  Opening a
// group (n mod 32 == 0) writes the channel's two pieces (the rest zero);
// otherwise one byte.
template <typename T>
__global__ void fp8_append_kernel(Planes p, const T* __restrict__ k, const T* __restrict__ v,
                                  int n)
{
    const int D = p.D;
    const int c = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (c >= D)
        return;
    const int g = n / G, j = n % G;
    const size_t blk = (bh * p.gcap + g) * (size_t)D * G;
    uint8_t* kd = reinterpret_cast<uint8_t*>(p.k_codes) + blk;
    uint8_t* vd = reinterpret_cast<uint8_t*>(p.v_codes) + blk;
    const uint32_t kb = fp8_e4m3(lde(k, bh * D + c));
    const uint32_t vb = fp8_e4m3(lde(v, bh * D + c));
    if (j == 0) {
        *reinterpret_cast<uint4*>(kd + fp8_offset(D, c, 0)) = make_uint4(kb, 0, 0, 0);
        *reinterpret_cast<uint4*>(kd + fp8_offset(D, c, 16)) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vd + fp8_offset(D, c, 0)) = make_uint4(vb, 0, 0, 0);
        *reinterpret_cast<uint4*>(vd + fp8_offset(D, c, 16)) = make_uint4(0, 0, 0, 0);
    } else {
        kd[fp8_offset(D, c, j)] = (uint8_t)kb;
        vd[fp8_offset(D, c, j)] = (uint8_t)vb;
    }
}

constexpr int kFp8Waves = 4;

// The 64 bytes of channels 2i and 2i+1 of one group: words 0..7 channel 2i
// (4 tokens each), 8..15 channel 2i+1; piece k (words 4k..4k+3) sits
// NP * 16 bytes after piece k-1.
struct Fp8Rows {
    uint32_t w[16];
};

template <int NP>
__device__ __forceinline__ void load_rows(const uint32_t* __restrict__ src, Fp8Rows& r)
{
    const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 v = s[k * NP];
        r.w[4 * k] = v.x;
        r.w[4 * k + 1] = v.y;
        r.w[4 * k + 2] = v.z;
        r.w[4 * k + 3] = v.w;
    }
}

// Tokens j, j+1 (j even) of one channel row (words w[0..7]).
template <int J>
__device__ __forceinline__ float2 fp8_pair(const uint32_t* w)
{
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(w[J / 4], ((J / 2) & 1) != 0);
    return make_float2(f[0], f[1]);
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kFp8Waves) void attend_fp8_kernel(
    Planes p, const T* __restrict__ q, float* __restrict__ out, int n, int splits)
{
    constexpr int NP = D / 2;
    __shared__ float red_m[kFp8Waves], red_l[kFp8Waves];
    __shared__ float red_o[kFp8Waves][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x;
    const size_t row = blockIdx.y;
    const int b = (int)(row / p.hq), h = (int)(row % p.hq);
    const size_t bh = (size_t)b * p.hkv + h / (p.hq / p.hkv);
    const bool act = lane < NP;
    const int i = act ? lane : 0;
    // conj of the rotated query pair, scaled by log2(e)/sqrt(D)
    float cqx, cqy;
    {
        const int pos = n - 1;
        const float2 rot = cmul(p.rope_group[(size_t)(pos / G) * NP + i],
                                p.rope_offset[(pos % G) * NP + i]);
        const float x = lde(q, row * D + 2 * i), y = lde(q, row * D + 2 * i + 1);
        const float sc = act ? kLog2e / sqrtf((float)D) : 0.f;
        cqx = (x * rot.x - y * rot.y) * sc;
        cqy = -(x * rot.y + y * rot.x) * sc;
    }
    // per-token twiddles e^{i j theta_i} inside a group, by recurrence from
    // the table's j = 0, 1, 16, 17 in steps of e^{2 i theta_i} (<= 8 steps)
    const float2 T1 = p.rope_offset[1 * NP + i], T2 = p.rope_offset[2 * NP + i];
    const float2 T16 = p.rope_offset[16 * NP + i], T17 = p.rope_offset[17 * NP + i];

    const int nchunks = (n + G - 1) / G;
    const int per = (nchunks + splits - 1) / splits;
    const int c0 = split * per;
    const int c1 = min(nchunks, c0 + per);
    const uint32_t* kbase = p.k_codes + bh * p.gcap * D * 8 + 4 * i;
    const uint32_t* vbase = p.v_codes + bh * p.gcap * D * 8 + 4 * i;
    float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;

    Fp8Rows kc;
    if (c0 + wave < c1)
        load_rows<NP>(kbase + (size_t)(c0 + wave) * D * 8, kc);
    for (int ch = c0 + wave; ch < c1; ch += kFp8Waves) {
        // this group's values (used after the scores and the softmax) and the
        // wave's next group of keys
        Fp8Rows vc, kn;
        load_rows<NP>(vbase + (size_t)ch * D * 8, vc);
        const bool more = ch + kFp8Waves < c1;
        if (more)
            load_rows<NP>(kbase + (size_t)(ch + kFp8Waves) * D * 8, kn);

        const int t0 = ch * G;
        const int cnt = min(G, n - t0);
        // P_j = conj(q') e^{i (gG + j) theta}: score term of token j = Re[P_j (x + i y)]
        const float2 rg = p.rope_group[(size_t)ch * NP + i];
        float2 P0 = make_float2(cqx * rg.x - cqy * rg.y, cqx * rg.y + cqy * rg.x);
        float2 P1 = cmul(P0, T1), P16 = cmul(P0, T16), P17 = cmul(P0, T17);
        // tokens J, J+1 and J+16, J+17; the first halving step (lanes 32..
        // keep token k+16) runs as soon as both are known
        float sc[G / 2];
#define KVQ_FP8_SCORE4(J)                                                             \
        {                                                                             \
            const float2 xa = fp8_pair<J>(kc.w), ya = fp8_pair<J>(kc.w + 8);          \
            const float2 xb = fp8_pair<J + 16>(kc.w), yb = fp8_pair<J + 16>(kc.w + 8); \
            const float s0 = P0.x * xa.x - P0.y * ya.x, s1 = P1.x * xa.y - P1.y * ya.y; \
            const float s2 = P16.x * xb.x - P16.y * yb.x;                             \
            const float s3 = P17.x * xb.y - P17.y * yb.y;                             \
            P0 = cmul(P0, T2);                                                        \
            P1 = cmul(P1, T2);                                                        \
            P16 = cmul(P16, T2);                                                      \
            P17 = cmul(P17, T2);                                                      \
            const auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0),     \
                                                             __float_as_uint(s2), false, false); \
            sc[J] = __uint_as_float(r0[0]) + __uint_as_float(r0[1]);                  \
            const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1),     \
                                                             __float_as_uint(s3), false, false); \
            sc[J + 1] = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);              \
        }
        KVQ_FP8_SCORE4(0) KVQ_FP8_SCORE4(2) KVQ_FP8_SCORE4(4) KVQ_FP8_SCORE4(6)
        KVQ_FP8_SCORE4(8) KVQ_FP8_SCORE4(10) KVQ_FP8_SCORE4(12) KVQ_FP8_SCORE4(14)
#undef KVQ_FP8_SCORE4
        // ---- the rest of the sum over the wave's 64 lanes
#pragma unroll
        for (int k = 0; k < 8; ++k) {  // across row pairs: odd rows keep k+8
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(sc[k]),
                                                            __float_as_uint(sc[k + 8]), false,
                                                            false);
            sc[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        {
            const bool up = (lane & 8) != 0;  // mirror inside a row: upper 8 keep k+4
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float send = up ? sc[k] : sc[k + 4];
                const float keep = up ? sc[k + 4] : sc[k];
                sc[k] = keep + dpp<kDppMirror>(send);
            }
        }
        {
            const bool up = (lane & 4) != 0;  // mirror inside 8 lanes: upper 4 keep k+2
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float send = up ? sc[k] : sc[k + 2];
                const float keep = up ? sc[k + 2] : sc[k];
                sc[k] = keep + dpp<kDppHalfMirror>(send);
            }
        }
        {
            const bool up = (lane & 2) != 0;
            const float send = up ? sc[0] : sc[1];
            const float keep = up ? sc[1] : sc[0];
            sc[0] = keep + dpp<kDppXor2>(send);
        }
        const float s = sc[0] + dpp<kDppXor1>(sc[0]);  // token lane/2, in log2 units

        // ---- online softmax over the group
        const float sv = (lane >> 1) < cnt ? s : -INFINITY;
        const float mn = fmaxf(m, wave_max<false>(sv));
        const float f = exp2f(m - mn);
        const float pj = exp2f(sv - mn);
        l = l * f + 0.5f * wave_sum(pj);  // every token sits in two lanes
        a0 *= f;
        a1 *= f;
        m = mn;

        // ---- values of pair i, weighted (weight 0 past n; bytes there are 0)
#define KVQ_FP8_VALUE(J)                                                              \
        {                                                                             \
            const float2 xs = fp8_pair<J>(vc.w);                                      \
            const float2 ys = fp8_pair<J>(vc.w + 8);                                  \
            const float p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), 2 * J)); \
            const float p1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), 2 * J + 2)); \
            a0 = fmaf(p0, xs.x, a0);                                                  \
            a1 = fmaf(p0, ys.x, a1);                                                  \
            a0 = fmaf(p1, xs.y, a0);                                                  \
            a1 = fmaf(p1, ys.y, a1);                                                  \
        }
        KVQ_FP8_VALUE(0) KVQ_FP8_VALUE(2) KVQ_FP8_VALUE(4) KVQ_FP8_VALUE(6)
        KVQ_FP8_VALUE(8) KVQ_FP8_VALUE(10) KVQ_FP8_VALUE(12) KVQ_FP8_VALUE(14)
        KVQ_FP8_VALUE(16) KVQ_FP8_VALUE(18) KVQ_FP8_VALUE(20) KVQ_FP8_VALUE(22)
        KVQ_FP8_VALUE(24) KVQ_FP8_VALUE(26) KVQ_FP8_VALUE(28) KVQ_FP8_VALUE(30)
#undef KVQ_FP8_VALUE
        if (more)
            kc = kn;
    }

    // ---- merge the waves; one split writes the output, several write partials
    if (lane == 0) {
        red_m[wave] = m;
        red_l[wave] = l;
    }
    if (act) {
        red_o[wave][2 * i] = a0;
        red_o[wave][2 * i + 1] = a1;
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kFp8Waves; ++w)
            M = fmaxf(M, red_m[w]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kFp8Waves; ++w) {
            if (red_m[w] == -INFINITY)
                continue;
            const float fw = exp2f(red_m[w] - M);
            L += fw * red_l[w];
            o += fw * red_o[w][c];
        }
        if (splits == 1) {
            out[row * D + c] = o / L;
        } else {
            float* dst = p.partials + (row * p.max_splits + split) * (D + 2);
            dst[c] = o;
            if (c == 0) {
                dst[D] = M;
                dst[D + 1] = L;
            }
        }
    }
}

template <typename T>
hipError_t fp8_prefill_t(const Planes& p, const T* k, const T* v, int n, hipStream_t s)
{
    const int groups = (n + G - 1) / G;
    const int gpb = 256 / p.D;
    dim3 grid((groups + gpb - 1) / gpb, p.nb * p.hkv);
    fp8_prefill_kernel<T><<<grid, gpb * p.D, 0, s>>>(p.k_codes, k, n, groups, p.gcap, p.D);
    fp8_prefill_kernel<T><<<grid, gpb * p.D, 0, s>>>(p.v_codes, v, n, groups, p.gcap, p.D);
    return hipGetLastError();
}

template <typename T, int D>
void attend_fp8_t(const Planes& p, const void* q, float* out, int n, int splits, hipStream_t s)
{
    dim3 grid(splits, p.nb * p.hq);
    attend_fp8_kernel<T, D><<<grid, 64 * kFp8Waves, 0, s>>>(p, static_cast<const T*>(q), out, n,
                                                           splits);
    if (splits > 1)
        combine_kernel<D><<<p.nb * p.hq, D, 0, s>>>(p.partials, p.max_splits, splits, out);
}

}  // namespace

hipError_t launch_fp8_prefill(const Planes& p, const void* k, const void* v, int n,
                              hipStream_t s)
{
    if (p.dtype == 0)
        return fp8_prefill_t<__half>(p, static_cast<const __half*>(k),
                                     static_cast<const __half*>(v), n, s);
    return fp8_prefill_t<float>(p, static_cast<const float*>(k), static_cast<const float*>(v), n,
                                s);
}

hipError_t launch_fp8_append(const Planes& p, const void* k, const void* v, int n, hipStream_t s)
{
    if (p.dtype == 0)
        fp8_append_kernel<__half><<<p.nb * p.hkv, p.D, 0, s>>>(
            p, static_cast<const __half*>(k), static_cast<const __half*>(v), n);
    else
        fp8_append_kernel<float><<<p.nb * p.hkv, p.D, 0, s>>>(
            p, static_cast<const float*>(k), static_cast<const float*>(v), n);
    return hipGetLastError();
}

hipError_t launch_attend_fp8(const Planes& p, const void* q, float* out, int n, int splits,
                             hipStream_t s)
{
    if (p.dtype == 0) {
        if (p.D == 64) attend_fp8_t<__half, 64>(p, q, out, n, splits, s);
        else attend_fp8_t<__half, 128>(p, q, out, n, splits, s);
    } else {
        if (p.D == 64) attend_fp8_t<float, 64>(p, q, out, n, splits, s);
        else attend_fp8_t<float, 128>(p, q, out, n, splits, s);
    }
    return hipGetLastError();
}

}  // namespace kvqi
