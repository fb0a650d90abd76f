// kvq_geometry.hip -- gfx950 kernels for the geometry ablation and for the
// error of a cache measured where it is consumed.
//
// Geometry ablation ("Your KV Cache Doesn't Have a Bit Problem...", lede and
// sections "Keys: The Outliers Live in Fixed Channels", "Values: Where the
// Intuition Breaks"): the same bits spent along the other axis -- keys
// grouped per token (G channels of one token) and/or values grouped per
// channel (one channel over G tokens).  A flipped operand takes the other
// operand's plane layout, so its attention reads keys token-major or values
// channel-major; this kernel does that plainly (it is the comparison point,
// not the tuned path): lane = channel pair, 32-token chunks per wave, the 64
// partial scores of a chunk summed by a lane-halving shuffle reduction, online
// softmax in log2 units, (o, m, l) partials merged by the main path's combine
// kernel.
//
// Error where it is consumed (same page, "Values: Where the Intuition
// Breaks": validate on the attention output, not on the stored tensor): per
// output row, in fp64, softmax weights from the unquantized and from the
// stored keys, the reference output, the output with stored values and the
// end-to-end output, and the reconstruction errors of the row's KV head.
#include "kvq_attend_kernel.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>
#include <math.h>

namespace kvqi {
namespace {

template <typename T> __device__ __forceinline__ float ldf(const T* p, size_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<__half>(const __half* p, size_t i)
{
    return __half2float(p[i]);
}

// zero + step * code with the binary16 step in bits 0..15 and zero in 16..31
__device__ __forceinline__ float deq(uint32_t meta, uint32_t code)
{
    return fmaf(h2f(meta), (float)code, h2f(meta >> 16));
}

__device__ __forceinline__ float lane_value(float v, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

constexpr int kGeoWaves = 4;

// Grid (splits, batch * q_heads); 4 waves.  Split s takes 32-token chunks
// [s * per, (s + 1) * per); its waves take them in turn.
template <typename T, int D, int KB, int VB, int GEOM>
__global__ __launch_bounds__(64 * kGeoWaves) void attend_geometry_kernel(
    Planes p, const T* __restrict__ q, float* __restrict__ out, int n, int splits)
{
    constexpr int NP = D / 2;
    constexpr int WK = G * KB / 32, WV = G * VB / 32;
    constexpr uint32_t KMASK = (1u << KB) - 1, VMASK = (1u << VB) - 1;
    constexpr bool KTOK = (GEOM & kKeysPerToken) != 0;
    constexpr bool VCH = (GEOM & kValuesPerChannel) != 0;
    __shared__ float2 tw[G * NP];
    __shared__ float red_m[kGeoWaves], red_l[kGeoWaves];
    __shared__ float red_o[kGeoWaves][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x;
    const size_t row = blockIdx.y;
    const int b = (int)(row / p.hq), h = (int)(row % p.hq);
    const size_t bh = (size_t)b * p.hkv + h / (p.hq / p.hkv);
    for (int x = threadIdx.x; x < G * NP; x += blockDim.x)
        tw[x] = p.rope_offset[x];

    const bool act = lane < NP;
    const int i = act ? lane : 0;
    float qx, qy;
    {
        const int pos = n - 1;
        const float2 rg = p.rope_group[(size_t)(pos / G) * NP + i];
        const float2 ro = p.rope_offset[(pos % G) * NP + i];
        const float c = rg.x * ro.x - rg.y * ro.y, s = rg.x * ro.y + rg.y * ro.x;
        const float x = ldf(q, row * D + 2 * i), y = ldf(q, row * D + 2 * i + 1);
        qx = act ? x * c - y * s : 0.f;
        qy = act ? x * s + y * c : 0.f;
    }
    const float scale = kLog2e / sqrtf((float)D);
    __syncthreads();

    const int nchunks = (n + G - 1) / G;
    const int per = (nchunks + splits - 1) / splits;
    const int c0 = split * per;
    const int c1 = min(nchunks, c0 + per);
    const int tq = n / G * G;  // an operand grouped per channel is quantized below
    const T* ktail = reinterpret_cast<const T*>(p.k_tail) + bh * p.ring * D;
    const T* vtail = reinterpret_cast<const T*>(p.v_tail) + bh * p.ring * D;
    float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
    int tw_base = i;  // made opaque per chunk: the twiddle reads stay in the loop

    // Tokens past n in the last chunk read token n-1 (in bounds) and get
    // weight 0, so every chunk runs the same branch-free token loops.
    for (int ch = c0 + wave; ch < c1; ch += kGeoWaves) {
        asm volatile("" : "+v"(tw_base));
        const int t0 = ch * G;
        const int cnt = min(G, n - t0);
        const float2 rg = p.rope_group[(size_t)ch * NP + i];
        float sc[G];
        auto score = [&](int j, float x, float y) {
            const float2 ro = tw[j * NP + tw_base];
            const float c = rg.x * ro.x - rg.y * ro.y, s = rg.x * ro.y + rg.y * ro.x;
            sc[j] = qx * (x * c - y * s) + qy * (x * s + y * c);
        };

        // ---- keys: partial score of pair i for the chunk's tokens
        if (KTOK) {
            uint32_t mt[G], wd[G];
            const int e = ((2 * i) % G) * KB;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int t = min(t0 + j, n - 1);
                const size_t tc = (bh * p.tcap + t) * (D / G) + (2 * i) / G;
                mt[j] = p.k_meta[tc];
                wd[j] = p.k_codes[tc * WK + e / 32];
            }
#pragma unroll
            for (int j = 0; j < G; ++j)
                score(j, deq(mt[j], (wd[j] >> (e % 32)) & KMASK),
                      deq(mt[j], (wd[j] >> (e % 32 + KB)) & KMASK));
        } else if (t0 + G <= tq) {
            const size_t gc = (bh * p.gcap + ch) * D + 2 * i;
            const uint32_t km0 = p.k_meta[gc], km1 = p.k_meta[gc + 1];
            uint32_t kw[2 * WK];
#pragma unroll
            for (int w = 0; w < 2 * WK; ++w)
                kw[w] = p.k_codes[gc * WK + w];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int e = j * KB;
                score(j, deq(km0, (kw[e / 32] >> (e % 32)) & KMASK),
                      deq(km1, (kw[WK + e / 32] >> (e % 32)) & KMASK));
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const T* r = ktail + (size_t)(min(t0 + j, n - 1) % p.ring) * D + 2 * i;
                score(j, ldf(r, 0), ldf(r, 1));
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
            sc[j] = act ? sc[j] : 0.f;
        // sum over the 64 lanes: each step halves the vector between lane
        // pairs; afterwards lane L holds the score of token L mod 32
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) {
            const bool up = (lane & o) != 0;
#pragma unroll
            for (int k = 0; k < o; ++k) {
                const float send = up ? sc[k] : sc[k + o];
                const float keep = up ? sc[k + o] : sc[k];
                sc[k] = keep + __shfl_xor(send, o);
            }
        }
        const float sum = sc[0] + __shfl_xor(sc[0], 32);

        // ---- online softmax over the chunk (log2 units)
        const float sv = (lane & 31) < cnt ? sum * scale : -INFINITY;
        float cm = sv;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1)
            cm = fmaxf(cm, __shfl_xor(cm, o));
        const float mn = fmaxf(m, cm);
        const float f = exp2f(m - mn);
        const float pj = exp2f(sv - mn);
        float ps = pj;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1)
            ps += __shfl_xor(ps, o);
        l = l * f + ps;
        a0 *= f;
        a1 *= f;
        m = mn;

        // ---- values: pair i of each token, weighted (weight 0 past n)
        auto acc = [&](int j, float x, float y) {
            const float wj = lane_value(pj, j);
            a0 = fmaf(wj, x, a0);
            a1 = fmaf(wj, y, a1);
        };
        if (!VCH) {
            uint32_t mt[G], wd[G];
            const int e = ((2 * i) % G) * VB;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int t = min(t0 + j, n - 1);
                const size_t tc = (bh * p.tcap + t) * (D / G) + (2 * i) / G;
                mt[j] = p.v_meta[tc];
                wd[j] = p.v_codes[tc * WV + e / 32];
            }
#pragma unroll
            for (int j = 0; j < G; ++j)
                acc(j, deq(mt[j], (wd[j] >> (e % 32)) & VMASK),
                    deq(mt[j], (wd[j] >> (e % 32 + VB)) & VMASK));
        } else if (t0 + G <= tq) {
            const size_t gc = (bh * p.gcap + ch) * D + 2 * i;
            const uint32_t vm0 = p.v_meta[gc], vm1 = p.v_meta[gc + 1];
            uint32_t vw[2 * WV];
#pragma unroll
            for (int w = 0; w < 2 * WV; ++w)
                vw[w] = p.v_codes[gc * WV + w];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int e = j * VB;
                acc(j, deq(vm0, (vw[e / 32] >> (e % 32)) & VMASK),
                    deq(vm1, (vw[WV + e / 32] >> (e % 32)) & VMASK));
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const T* r = vtail + (size_t)(min(t0 + j, n - 1) % p.ring) * D + 2 * i;
                acc(j, ldf(r, 0), ldf(r, 1));
            }
        }
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
        for (int w = 0; w < kGeoWaves; ++w)
            M = fmaxf(M, red_m[w]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kGeoWaves; ++w) {
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

template <typename T, int D, int KB, int VB>
void geo_launch(const Planes& p, const void* q, float* out, int n, int splits, hipStream_t s)
{
    dim3 grid(splits, p.nb * p.hq);
    const T* qt = static_cast<const T*>(q);
    switch (p.geometry) {
    case 1: attend_geometry_kernel<T, D, KB, VB, 1><<<grid, 64 * kGeoWaves, 0, s>>>(p, qt, out, n, splits); break;
    case 2: attend_geometry_kernel<T, D, KB, VB, 2><<<grid, 64 * kGeoWaves, 0, s>>>(p, qt, out, n, splits); break;
    case 3: attend_geometry_kernel<T, D, KB, VB, 3><<<grid, 64 * kGeoWaves, 0, s>>>(p, qt, out, n, splits); break;
    }
    if (splits > 1)
        combine_kernel<D><<<p.nb * p.hq, D, 0, s>>>(p.partials, p.max_splits, splits, out);
}

template <typename T, int D, int KB>
void geo_vb(const Planes& p, const void* q, float* out, int n, int splits, hipStream_t s)
{
    switch (p.vbits) {
    case 2: geo_launch<T, D, KB, 2>(p, q, out, n, splits, s); break;
    case 4: geo_launch<T, D, KB, 4>(p, q, out, n, splits, s); break;
    case 8: geo_launch<T, D, KB, 8>(p, q, out, n, splits, s); break;
    }
}

template <typename T, int D>
void geo_kb(const Planes& p, const void* q, float* out, int n, int splits, hipStream_t s)
{
    switch (p.kbits) {
    case 2: geo_vb<T, D, 2>(p, q, out, n, splits, s); break;
    case 4: geo_vb<T, D, 4>(p, q, out, n, splits, s); break;
    case 8: geo_vb<T, D, 8>(p, q, out, n, splits, s); break;
    }
}

// ------------------------------------------------------------- metrics --

// Element (t, c) of one operand as the cache stores it, in fp64: a sink row,
// a dequantized code (grouped per token: [tcap][D/G][W]; per channel:
// [gcap][D][W]), or a verbatim tail/ring row.  Grouped per token, tokens at
// or above tq are quantized too unless `ring_values` (a residual window on
// the values) holds them in the ring.
template <typename T>
__device__ double stored_elem(const Planes& p, bool per_token, bool ring_values, int bits,
                              const uint32_t* codes, const uint32_t* meta, const void* ring,
                              const void* sink, size_t bh, int t, int c, int ns, int tq)
{
    const int D = p.D;
    if (t < ns)
        return (double)ldf(reinterpret_cast<const T*>(sink), (bh * p.sink + t) * D + c);
    const int W = G * bits / 32;
    const uint32_t mask = (1u << bits) - 1;
    if (per_token && (!ring_values || t < tq)) {
        const size_t tc = (bh * p.tcap + t) * (D / G) + c / G;
        const int e = (c % G) * bits;
        const uint32_t mt = meta[tc];
        const uint32_t code = (codes[tc * W + e / 32] >> (e % 32)) & mask;
        return (double)h2f(mt >> 16) + (double)h2f(mt) * (double)code;
    }
    if (!per_token && t < tq) {
        const size_t gc = (bh * p.gcap + t / G) * D + c;
        const int e = (t % G) * bits;
        const uint32_t mt = meta[gc];
        const uint32_t code = (codes[gc * W + e / 32] >> (e % 32)) & mask;
        return (double)h2f(mt >> 16) + (double)h2f(mt) * (double)code;
    }
    return (double)ldf(reinterpret_cast<const T*>(ring), (bh * p.ring + t % p.ring) * D + c);
}

// Sum (or max) over the block's 256 threads; every thread gets the result.
template <bool MAX>
__device__ double block_reduce(double x, double* buf)
{
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int s = blockDim.x / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s)
            buf[threadIdx.x] = MAX ? fmax(buf[threadIdx.x], buf[threadIdx.x + s])
                                   : buf[threadIdx.x] + buf[threadIdx.x + s];
        __syncthreads();
    }
    const double r = buf[0];
    __syncthreads();
    return r;
}

constexpr int kMetricThreads = 256;
constexpr int kMaxPairs = 64;

// One block per output row r = b * q_heads + h; writes 6 fp64 sums to rows[r]:
// sum (ahat - a)^2, |A vhat - A v|^2, |A v|^2, |Ahat vhat - A v|^2,
// sum (khat - k)^2 and sum (vhat - v)^2 (the last two over the KV head).
template <typename T>
__global__ __launch_bounds__(kMetricThreads) void metrics_rows_kernel(
    Planes p, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ q, int n,
    double* __restrict__ rows)
{
    __shared__ double th[kMaxPairs], qr[2 * kMaxPairs];
    __shared__ double wa[kMetricThreads], wh[kMetricThreads], buf[kMetricThreads];
    const int D = p.D, NP = D / 2, tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const int b = (int)(row / p.hq), h = (int)(row % p.hq);
    const size_t bh = (size_t)b * p.hkv + h / (p.hq / p.hkv);
    const bool ktok = (p.geometry & kKeysPerToken) != 0;
    const bool vtok = (p.geometry & kValuesPerChannel) == 0;
    const int ns = n < p.sink ? n : p.sink;
    const int tq = quantized_end(n, p.residual, p.sink);
    const bool vring = p.residual > 0;
    if (tid < NP) {
        const double theta = pow(p.rope_base, -2.0 * tid / (double)D);
        th[tid] = theta;
        double sn, cs;
        sincos((double)(n - 1) * theta, &sn, &cs);
        const double x = ldf(q, row * D + 2 * tid), y = ldf(q, row * D + 2 * tid + 1);
        qr[2 * tid] = x * cs - y * sn;
        qr[2 * tid + 1] = x * sn + y * cs;
    }
    __syncthreads();
    const double rsd = 1.0 / sqrt((double)D);

    // scores of token t from the unquantized (s) and the stored keys (sh)
    auto scores = [&](int t, double& s, double& sh, double* kerr) {
        s = 0.0;
        sh = 0.0;
        const size_t base = (bh * n + t) * D;
        for (int pi = 0; pi < NP; ++pi) {
            double sn, cs;
            sincos((double)t * th[pi], &sn, &cs);
            const double x = ldf(k, base + 2 * pi), y = ldf(k, base + 2 * pi + 1);
            const double xh = stored_elem<T>(p, ktok, false, p.kbits, p.k_codes, p.k_meta,
                                             p.k_tail, p.k_sink, bh, t, 2 * pi, ns, tq);
            const double yh = stored_elem<T>(p, ktok, false, p.kbits, p.k_codes, p.k_meta,
                                             p.k_tail, p.k_sink, bh, t, 2 * pi + 1, ns, tq);
            if (kerr)
                *kerr += (xh - x) * (xh - x) + (yh - y) * (yh - y);
            s += qr[2 * pi] * (x * cs - y * sn) + qr[2 * pi + 1] * (x * sn + y * cs);
            sh += qr[2 * pi] * (xh * cs - yh * sn) + qr[2 * pi + 1] * (xh * sn + yh * cs);
        }
        s *= rsd;
        sh *= rsd;
    };

    // pass 1: per-thread online (max, sum) for both weight sets and the
    // reconstruction errors
    double m = -INFINITY, l = 0.0, mh = -INFINITY, lh = 0.0, kerr = 0.0, verr = 0.0;
    for (int t = tid; t < n; t += kMetricThreads) {
        double s, sh;
        scores(t, s, sh, &kerr);
        if (s > m) {
            l = l * exp(m - s) + 1.0;
            m = s;
        } else {
            l += exp(s - m);
        }
        if (sh > mh) {
            lh = lh * exp(mh - sh) + 1.0;
            mh = sh;
        } else {
            lh += exp(sh - mh);
        }
        for (int c = 0; c < D; ++c) {
            const double x = ldf(v, (bh * n + t) * D + c);
            const double xh = stored_elem<T>(p, vtok, vring, p.vbits, p.v_codes, p.v_meta,
                                             p.v_tail, p.v_sink, bh, t, c, ns, tq);
            verr += (xh - x) * (xh - x);
        }
    }
    const double M = block_reduce<true>(m, buf);
    const double L = block_reduce<false>(m == -INFINITY ? 0.0 : l * exp(m - M), buf);
    const double Mh = block_reduce<true>(mh, buf);
    const double Lh = block_reduce<false>(mh == -INFINITY ? 0.0 : lh * exp(mh - Mh), buf);

    // pass 2: tiles of 256 tokens; weights to LDS, then channel threads sum
    double serr = 0.0, o_ref = 0.0, o_vq = 0.0, o_e2e = 0.0;
    for (int t0 = 0; t0 < n; t0 += kMetricThreads) {
        const int t = t0 + tid;
        double a = 0.0, ah = 0.0;
        if (t < n) {
            double s, sh;
            scores(t, s, sh, nullptr);
            a = exp(s - M) / L;
            ah = exp(sh - Mh) / Lh;
            serr += (ah - a) * (ah - a);
        }
        wa[tid] = a;
        wh[tid] = ah;
        __syncthreads();
        if (tid < D) {
            const int cnt = n - t0 < kMetricThreads ? n - t0 : kMetricThreads;
            for (int j = 0; j < cnt; ++j) {
                const double x = ldf(v, (bh * n + t0 + j) * D + tid);
                const double xh = stored_elem<T>(p, vtok, vring, p.vbits, p.v_codes, p.v_meta,
                                                 p.v_tail, p.v_sink, bh, t0 + j, tid, ns, tq);
                o_ref += wa[j] * x;
                o_vq += wa[j] * xh;
                o_e2e += wh[j] * xh;
            }
        }
        __syncthreads();
    }
    const double r0 = block_reduce<false>(serr, buf);
    const double r1 = block_reduce<false>((o_vq - o_ref) * (o_vq - o_ref), buf);
    const double r2 = block_reduce<false>(o_ref * o_ref, buf);
    const double r3 = block_reduce<false>((o_e2e - o_ref) * (o_e2e - o_ref), buf);
    const double r4 = block_reduce<false>(kerr, buf);
    const double r5 = block_reduce<false>(verr, buf);
    if (tid == 0) {
        double* dst = rows + row * 6;
        dst[0] = r0;
        dst[1] = r1;
        dst[2] = r2;
        dst[3] = r3;
        dst[4] = r4;
        dst[5] = r5;
    }
}

// The five metrics: means over the rows of sqrt(sum (khat-k)^2),
// sqrt(sum (ahat-a)^2), sqrt(sum (vhat-v)^2), |A vhat - A v| / |A v| and
// |Ahat vhat - A v| / |A v|.  One block.
__global__ __launch_bounds__(kMetricThreads) void metrics_final_kernel(
    const double* __restrict__ rows, int nrows, double* __restrict__ metrics)
{
    __shared__ double buf[kMetricThreads];
    double acc[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int r = threadIdx.x; r < nrows; r += kMetricThreads) {
        const double* x = rows + (size_t)r * 6;
        acc[0] += sqrt(x[4]);
        acc[1] += sqrt(x[0]);
        acc[2] += sqrt(x[5]);
        acc[3] += sqrt(x[1] / x[2]);
        acc[4] += sqrt(x[3] / x[2]);
    }
    for (int i = 0; i < 5; ++i) {
        const double s = block_reduce<false>(acc[i], buf);
        if (threadIdx.x == 0)
            metrics[i] = s / nrows;
    }
}

}  // namespace

hipError_t launch_attend_geometry(const Planes& p, const void* q, float* out, int n, int splits,
                                  hipStream_t s)
{
    if (p.dtype == 0) {
        if (p.D == 64) geo_kb<__half, 64>(p, q, out, n, splits, s);
        else geo_kb<__half, 128>(p, q, out, n, splits, s);
    } else {
        if (p.D == 64) geo_kb<float, 64>(p, q, out, n, splits, s);
        else geo_kb<float, 128>(p, q, out, n, splits, s);
    }
    return hipGetLastError();
}

hipError_t launch_error_metrics(const Planes& p, const void* k, const void* v, const void* q,
                                double* metrics, int n, hipStream_t s)
{
    // per-row sums in the partials region: rows * 6 doubles fit in
    // rows * max_splits * (D + 2) floats
    double* rows = reinterpret_cast<double*>(p.partials);
    const int nrows = p.nb * p.hq;
    if (p.dtype == 0)
        metrics_rows_kernel<__half><<<nrows, kMetricThreads, 0, s>>>(
            p, static_cast<const __half*>(k), static_cast<const __half*>(v),
            static_cast<const __half*>(q), n, rows);
    else
        metrics_rows_kernel<float><<<nrows, kMetricThreads, 0, s>>>(
            p, static_cast<const float*>(k), static_cast<const float*>(v),
            static_cast<const float*>(q), n, rows);
    metrics_final_kernel<<<1, kMetricThreads, 0, s>>>(rows, nrows, metrics);
    return hipGetLastError();
}

}  // namespace kvqi
