// kvq_kernels.hip -- gfx950 kernels: key/value quantize-and-pack and the
// key-tail append and flush (decode attention lives in kvq_attend_kernel.h,
// instantiated by kvq_attend_d64.hip and kvq_attend_d128.hip).
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
#include "kvq_append.h"
#include "kvq_codec.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace kvqi {
namespace {

constexpr int G = kGroup;

// ------------------------------------------------------------- binary16 --

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return __half2float(__ushort_as_half((unsigned short)h));
}

// ------------------------------------------------------- prefill kernels --

// Key groups per 256-thread block: a thread takes one channel of a group
// (fp32 inputs) or two adjacent channels (binary16 inputs: one 32-bit load
// per token, both channels' statistics on packed pairs).
template <typename T>
__host__ __device__ constexpr int key_groups_per_block(int D)
{
    return std::is_same<T, __half>::value ? 512 / D : 256 / D;
}

// One thread per (sequence*head, key group, channel or channel pair): walks
// the group's G tokens down the channel, so the per-channel statistics need
// no cross-lane reduction; consecutive threads read consecutive channels of
// a token row.  Block bx of sequence/head bh covers key groups
// g_begin + bx * key_groups_per_block .. ; per-sequence bases are uniform,
// per-thread offsets 32-bit (a sequence/head holds under 2^31 elements).
template <typename T, int BITS, int D>
__device__ __forceinline__ void quant_keys_block(const Planes& p, const T* __restrict__ k,
                                                 int n_tokens, int g_begin, int g_end, int bx,
                                                 size_t bh)
{
    constexpr int WK = G * BITS / 32;
    const T* kb = k + bh * (size_t)n_tokens * D;
    uint32_t* cb = p.k_codes + bh * (size_t)p.gcap * D * WK;
    uint32_t* mb = p.k_meta + bh * (size_t)p.gcap * D;
    if constexpr (std::is_same<T, __half>::value) {
        constexpr int np = D / 2;  // channel pairs
        const int cp = threadIdx.x % np;
        const int g = g_begin + bx * key_groups_per_block<T>(D) + threadIdx.x / np;
        if (g >= g_end)
            return;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(kb) + (uint32_t)(g * G * np + cp);
        uint32_t d[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            d[j] = src[j * np];
        uint32_t w0[WK], w1[WK], m0, m1;
        quantize_group_two<BITS>(d, w0, w1, m0, m1);
        const uint32_t gc = (uint32_t)(g * D + 2 * cp);  // channel 2cp; 2cp+1 follows
        uint32_t* dst = cb + gc * WK;
#pragma unroll
        for (int i = 0; i < WK; ++i) {
            dst[i] = w0[i];
            dst[WK + i] = w1[i];
        }
        *reinterpret_cast<uint2*>(mb + gc) = make_uint2(m0, m1);
        return;
    }
    constexpr int gpb = 256 / D;
    const int c = threadIdx.x % D;
    const int g = g_begin + bx * gpb + threadIdx.x / D;
    if (g >= g_end)
        return;
    const T* src = kb + (uint32_t)(g * G * D + c);
    float x[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        x[j] = to_f32(src[j * D]);
    uint32_t w[WK];
    const uint32_t meta = quantize_group<BITS>(x, w);
    const uint32_t gc = (uint32_t)(g * D + c);
    uint32_t* dst = cb + gc * WK;
#pragma unroll
    for (int i = 0; i < WK; ++i)
        dst[i] = w[i];
    mb[gc] = meta;
}

template <typename T, int BITS, int D>
__global__ __launch_bounds__(256) void quant_keys_kernel(Planes p, const T* __restrict__ k,
                                                         int n_tokens, int g_begin, int g_end)
{
    quant_keys_block<T, BITS, D>(p, k, n_tokens, g_begin, g_end, blockIdx.x, blockIdx.y);
}

// Copy tokens [t0, t1) of each sequence/head verbatim into a buffer of
// `slots` token rows per sequence/head, token t in slot t mod slots (the
// tail rings, or the sinks with slots = S > t).
template <typename T>
__global__ void copy_tail_kernel(Planes p, const T* __restrict__ src, T* __restrict__ dst,
                                 int slots, int n_tokens, int t0, int t1, size_t total)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int D = p.D;
    const int rem = t1 - t0;
    const int c = idx % D;
    const int t = t0 + (int)((idx / D) % rem);
    const size_t bh = idx / ((size_t)D * rem);
    dst[(bh * slots + t % slots) * D + c] = src[(bh * n_tokens + t) * D + c];
}

// Value groups per 256-thread block row: block bx of sequence/head bh takes
// the groups (token t, channel group cg) with t * (D/G) + cg in
// [256 bx, 256 bx + 256).
__host__ __device__ constexpr int value_blocks(int n_src, int D)
{
    return (n_src * (D / G) + 255) / 256;
}

// One thread per (sequence*head, token, channel group): the group is G
// consecutive channels of one token row (64 contiguous bytes at fp16).
// Input tokens [0, n_src) of rows of src_stride tokens go to cache slots
// [t_dst0, t_dst0 + n_src); the thread's group is number
// 256 bx + threadIdx.x of sequence/head bh.
template <typename T, int BITS, int D>
__device__ __forceinline__ void quant_values_thread(const Planes& p, const T* __restrict__ v,
                                                    int n_src, int src_stride, int t_dst0, int bx,
                                                    size_t bh)
{
    constexpr int WV = G * BITS / 32;
    constexpr int cg_bits = D == 128 ? 2 : 1;  // D / G = 4 or 2 channel groups
    const uint32_t local = (uint32_t)bx * 256u + threadIdx.x;
    if (local >= (uint32_t)n_src << cg_bits)
        return;
    const uint32_t t = local >> cg_bits, cg = local & ((1u << cg_bits) - 1u);
    const T* src = v + bh * (size_t)src_stride * D + (t * (uint32_t)D + cg * G);
    const size_t row0 = bh * (size_t)p.tcap + t_dst0;  // first destination token row
    uint32_t* dst = p.v_codes + (row0 << cg_bits) * WV + local * WV;
    uint32_t* mdst = p.v_meta + (row0 << cg_bits) + local;
    uint32_t w[WV];
    uint32_t meta;
    if constexpr (std::is_same<T, __half>::value) {
        // 64 contiguous bytes (16-byte aligned: rows of D >= 64 binary16)
        uint32_t d[G / 2];
#pragma unroll
        for (int i = 0; i < G / 8; ++i) {
            const uint4 q = reinterpret_cast<const uint4*>(src)[i];
            d[4 * i] = q.x;
            d[4 * i + 1] = q.y;
            d[4 * i + 2] = q.z;
            d[4 * i + 3] = q.w;
        }
        meta = quantize_group_pairs<BITS>(d, w);
    } else {
        float x[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            x[j] = to_f32(src[j]);
        meta = quantize_group<BITS>(x, w);
    }
#pragma unroll
    for (int i = 0; i < WV; ++i)
        dst[i] = w[i];
    *mdst = meta;
}

// grid (value_blocks(n_src, D), sequences/heads in this launch); bh0 = the
// first sequence/head
template <typename T, int BITS, int D>
__global__ __launch_bounds__(256) void quant_values_kernel(Planes p, const T* __restrict__ v,
                                                           int n_src, int src_stride, int t_dst0,
                                                           size_t bh0)
{
    quant_values_thread<T, BITS, D>(p, v, n_src, src_stride, t_dst0, blockIdx.x,
                                    bh0 + blockIdx.y);
}

// Keys and values of a prefill in one launch: blocks [0, kblocks) run the
// key codec (block kb: key-group block kb % kgx of sequence/head kb / kgx),
// the rest the value codec (value block vb % vbx of sequence/head vb / vbx,
// vb = block - kblocks).  Keys first, then values: on the Llama-2-7B-shaped
// prompt (8 x 32 heads x 4095 tokens x 128, fp16) this measured 121 us
// against 133 us with key and value blocks alternating and 128 us as two
// launches; the one launch lets the last key blocks overlap the first value
// blocks.
template <typename T, int KB, int VB, int D>
__global__ __launch_bounds__(256) void quant_kv_kernel(Planes p, const T* __restrict__ k,
                                                       int n_tokens, int g_begin, int g_end,
                                                       int kgx, unsigned kblocks,
                                                       const T* __restrict__ v, int n_src,
                                                       int t_dst0, int vbx)
{
    const unsigned b = blockIdx.x;
    if (b < kblocks) {
        quant_keys_block<T, KB, D>(p, k, n_tokens, g_begin, g_end, (int)(b % (unsigned)kgx),
                                   b / (unsigned)kgx);
    } else {
        const unsigned i = b - kblocks;
        quant_values_thread<T, VB, D>(p, v, n_src, n_tokens, t_dst0, (int)(i % (unsigned)vbx),
                                      i / (unsigned)vbx);
    }
}

// Append one token per sequence/head in one launch (block = one sequence/head,
// head_dim threads, thread c = channel c): the value is quantized per token
// at once, the key goes to the tail and its group is quantized when the tail
// fills.
template <typename T, int KBITS, int VBITS>
__global__ void append_kernel(Planes p, const T* __restrict__ k, const T* __restrict__ v, int n)
{
    const int D = p.D;
    const int c = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (c >= D)
        return;  // D is a multiple of 64: whole waves only
    if (n < p.sink) {  // the first tokens stay in the sinks
        reinterpret_cast<T*>(p.k_sink)[(bh * p.sink + n) * D + c] = k[bh * D + c];
        reinterpret_cast<T*>(p.v_sink)[(bh * p.sink + n) * D + c] = v[bh * D + c];
        return;
    }
    append_token_groups<T, VBITS>(p.v_codes, p.v_meta, p.tcap, v + bh * D, bh, n, c, D);
    append_channel_groups<T, KBITS>(p.k_codes, p.k_meta, p.gcap,
                                    reinterpret_cast<T*>(p.k_tail) + bh * p.ring * D,
                                    k[bh * D + c], bh, n, c, D);
}

// The same for the geometry ablation (no windows): each operand is appended
// the way its grouping axis needs.
template <typename T, int KBITS, int VBITS, int GEOM>
__global__ void append_geometry_kernel(Planes p, const T* __restrict__ k,
                                       const T* __restrict__ v, int n)
{
    const int D = p.D;
    const int c = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (c >= D)
        return;
    if (GEOM & kKeysPerToken)
        append_token_groups<T, KBITS>(p.k_codes, p.k_meta, p.tcap, k + bh * D, bh, n, c, D);
    else
        append_channel_groups<T, KBITS>(p.k_codes, p.k_meta, p.gcap,
                                        reinterpret_cast<T*>(p.k_tail) + bh * p.ring * D,
                                        k[bh * D + c], bh, n, c, D);
    if (GEOM & kValuesPerChannel)
        append_channel_groups<T, VBITS>(p.v_codes, p.v_meta, p.gcap,
                                        reinterpret_cast<T*>(p.v_tail) + bh * p.ring * D,
                                        v[bh * D + c], bh, n, c, D);
    else
        append_token_groups<T, VBITS>(p.v_codes, p.v_meta, p.tcap, v + bh * D, bh, n, c, D);
}

// Append with a residual window (R > 0): key and value of token n go to ring
// slot n mod (R+G).  When n+1-R reaches a positive multiple of G, block b =
// (n+1-R)/G - 1 (tokens bG .. bG+G-1, all older than the window) is quantized
// from the rings in the same launch: thread c codes key channel c of the
// block (one key group) and value group c of the block (token bG + c/(D/G),
// channel group c mod (D/G)).  The block's slots differ from slot n mod (R+G)
// (they are R .. R+G-1 tokens older), so no thread reads what another writes.
template <typename T, int KBITS, int VBITS>
__global__ void append_residual_kernel(Planes p, const T* __restrict__ k,
                                       const T* __restrict__ v, int n)
{
    constexpr int WK = G * KBITS / 32, WV = G * VBITS / 32;
    const int D = p.D;
    const int c = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (c >= D)
        return;
    if (n < p.sink) {  // the first tokens stay in the sinks
        reinterpret_cast<T*>(p.k_sink)[(bh * p.sink + n) * D + c] = k[bh * D + c];
        reinterpret_cast<T*>(p.v_sink)[(bh * p.sink + n) * D + c] = v[bh * D + c];
        return;
    }
    T* kring = reinterpret_cast<T*>(p.k_tail) + bh * p.ring * D;
    T* vring = reinterpret_cast<T*>(p.v_tail) + bh * p.ring * D;
    const int slot = n % p.ring;
    kring[slot * D + c] = k[bh * D + c];
    vring[slot * D + c] = v[bh * D + c];
    const int aged = n + 1 - p.residual;
    if (aged < G || aged % G != 0)
        return;
    const int b = aged / G - 1;
    if (b * G < p.sink)
        return;  // that block is in the sinks
    {
        float x[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            x[j] = to_f32(kring[((b * G + j) % p.ring) * D + c]);
        uint32_t w[WK];
        const uint32_t meta = quantize_group<KBITS>(x, w);
        const size_t gc = (bh * p.gcap + b) * D + c;
#pragma unroll
        for (int i = 0; i < WK; ++i)
            p.k_codes[gc * WK + i] = w[i];
        p.k_meta[gc] = meta;
    }
    {
        const int ncg = D / G;
        const int t = b * G + c / ncg, cg = c % ncg;
        const T* src = vring + (size_t)(t % p.ring) * D + cg * G;
        float x[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            x[j] = to_f32(src[j]);
        uint32_t w[WV];
        const uint32_t meta = quantize_group<VBITS>(x, w);
        const size_t tc = (bh * p.tcap + t) * ncg + cg;
#pragma unroll
        for (int i = 0; i < WV; ++i)
            p.v_codes[tc * WV + i] = w[i];
        p.v_meta[tc] = meta;
    }
}

// ------------------------------------------------------------- dispatch --

// The key codec over channel groups [g_begin, g_end) (grid: key-group
// blocks x sequences/heads) and the value codec over tokens [0, n_src) (rows
// of src_stride tokens from src) into slots [t_dst0, t_dst0 + n_src), for
// one head dimension and code width.
template <typename T, int D>
void launch_keys_d(const Planes& q, int bits, const T* src, int n_tokens, int g_begin, int g_end,
                   hipStream_t stream)
{
    constexpr int gpb = key_groups_per_block<T>(D);
    const dim3 grid((g_end - g_begin + gpb - 1) / gpb, q.nb * q.hkv);
    switch (bits) {
    case 2: quant_keys_kernel<T, 2, D><<<grid, 256, 0, stream>>>(q, src, n_tokens, g_begin, g_end); break;
    case 4: quant_keys_kernel<T, 4, D><<<grid, 256, 0, stream>>>(q, src, n_tokens, g_begin, g_end); break;
    case 8: quant_keys_kernel<T, 8, D><<<grid, 256, 0, stream>>>(q, src, n_tokens, g_begin, g_end); break;
    }
}

template <typename T, int D>
void launch_values_d(const Planes& q, int bits, const T* src, int n_src, int src_stride,
                     int t_dst0, hipStream_t stream)
{
    const int nbh = q.nb * q.hkv;  // at most 65535 sequences/heads per launch
    for (int bh0 = 0; bh0 < nbh; bh0 += 65535) {
        const dim3 grid(value_blocks(n_src, D), nbh - bh0 < 65535 ? nbh - bh0 : 65535);
        switch (bits) {
        case 2: quant_values_kernel<T, 2, D><<<grid, 256, 0, stream>>>(q, src, n_src, src_stride, t_dst0, (size_t)bh0); break;
        case 4: quant_values_kernel<T, 4, D><<<grid, 256, 0, stream>>>(q, src, n_src, src_stride, t_dst0, (size_t)bh0); break;
        case 8: quant_values_kernel<T, 8, D><<<grid, 256, 0, stream>>>(q, src, n_src, src_stride, t_dst0, (size_t)bh0); break;
        }
    }
}

// Channel groups [g_begin, g_end) of src into the planes `codes`/`meta`
// (laid out [gcap][D][W]) and token groups of n_src tokens into planes laid
// out [tcap][D/G][W]: the two quantize kernels, pointed at any plane pair.
template <typename T>
void quantize_channel_groups(Planes q, uint32_t* codes, uint32_t* meta, int bits, const T* src,
                             int n_tokens, int g_begin, int g_end, hipStream_t stream)
{
    if (g_end <= g_begin)
        return;
    q.k_codes = codes;
    q.k_meta = meta;
    if (q.D == 128)
        launch_keys_d<T, 128>(q, bits, src, n_tokens, g_begin, g_end, stream);
    else
        launch_keys_d<T, 64>(q, bits, src, n_tokens, g_begin, g_end, stream);
}

template <typename T>
void launch_token_groups(const Planes& q, int bits, const T* src, int n_src, int src_stride,
                         int t_dst0, hipStream_t stream)
{
    if (n_src <= 0)
        return;
    if (q.D == 128)
        launch_values_d<T, 128>(q, bits, src, n_src, src_stride, t_dst0, stream);
    else
        launch_values_d<T, 64>(q, bits, src, n_src, src_stride, t_dst0, stream);
}

template <typename T>
void quantize_token_groups(Planes q, uint32_t* codes, uint32_t* meta, int bits, const T* src,
                           int n_src, int src_stride, int t_dst0, hipStream_t stream)
{
    q.v_codes = codes;
    q.v_meta = meta;
    launch_token_groups<T>(q, bits, src, n_src, src_stride, t_dst0, stream);
}

template <typename T>
void copy_rows(const Planes& p, const T* src, void* dst, int slots, int n_tokens, int t0, int t1,
               hipStream_t stream)
{
    const size_t total = t1 > t0 ? (size_t)p.nb * p.hkv * (t1 - t0) * p.D : 0;
    if (total > 0)
        copy_tail_kernel<T><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
            p, src, static_cast<T*>(dst), slots, n_tokens, t0, t1, total);
}

// Prefill with a non-zero geometry (no windows): an operand grouped per
// channel gets groups [0, n/G) and its last n mod G tokens in its tail; one
// grouped per token gets every token.
template <typename T>
hipError_t quantize_prefill_geometry(const Planes& p, const T* k, const T* v, int n_tokens,
                                     hipStream_t stream)
{
    const int tq = n_tokens / G * G;
    if (p.geometry & kKeysPerToken) {
        quantize_token_groups<T>(p, p.k_codes, p.k_meta, p.kbits, k, n_tokens, n_tokens, 0, stream);
    } else {
        quantize_channel_groups<T>(p, p.k_codes, p.k_meta, p.kbits, k, n_tokens, 0, tq / G, stream);
        copy_rows<T>(p, k, p.k_tail, p.ring, n_tokens, tq, n_tokens, stream);
    }
    if (p.geometry & kValuesPerChannel) {
        quantize_channel_groups<T>(p, p.v_codes, p.v_meta, p.vbits, v, n_tokens, 0, tq / G, stream);
        copy_rows<T>(p, v, p.v_tail, p.ring, n_tokens, tq, n_tokens, stream);
    } else {
        quantize_token_groups<T>(p, p.v_codes, p.v_meta, p.vbits, v, n_tokens, n_tokens, 0, stream);
    }
    return hipGetLastError();
}

template <typename T, int D>
void launch_kv_d(const Planes& p, const T* k, int n_tokens, int g_begin, int g_end, int kgx,
                 unsigned kblocks, const T* vsrc, int n_src, int t_dst0, int vbx,
                 unsigned vblocks, hipStream_t stream)
{
    const unsigned blocks = kblocks + vblocks;
#define KVQ_KV(KBB, VBB)                                                                 \
    quant_kv_kernel<T, KBB, VBB, D><<<blocks, 256, 0, stream>>>(                         \
        p, k, n_tokens, g_begin, g_end, kgx, kblocks, vsrc, n_src, t_dst0, vbx)
    switch (p.kbits * 16 + p.vbits) {
    case 2 * 16 + 2: KVQ_KV(2, 2); break;
    case 2 * 16 + 4: KVQ_KV(2, 4); break;
    case 2 * 16 + 8: KVQ_KV(2, 8); break;
    case 4 * 16 + 2: KVQ_KV(4, 2); break;
    case 4 * 16 + 4: KVQ_KV(4, 4); break;
    case 4 * 16 + 8: KVQ_KV(4, 8); break;
    case 8 * 16 + 2: KVQ_KV(8, 2); break;
    case 8 * 16 + 4: KVQ_KV(8, 4); break;
    case 8 * 16 + 8: KVQ_KV(8, 8); break;
    }
#undef KVQ_KV
}

template <typename T>
hipError_t quantize_prefill_t(const Planes& p, const T* k, const T* v, int n_tokens,
                              hipStream_t stream)
{
    if (p.geometry != 0)
        return quantize_prefill_geometry<T>(p, k, v, n_tokens, stream);
    // sink [0, ns), quantized [S, tq), rings [tq, n_tokens)
    const int ns = n_tokens < p.sink ? n_tokens : p.sink;
    const int tq = quantized_end(n_tokens, p.residual, p.sink);
    const int g_begin = p.sink / G, g_end = tq / G;
    const int nbh = p.nb * p.hkv;
    // values: every token from S on quantized without a window; with one,
    // [S, tq) quantized and the rest copied to the value ring
    const int vq = p.residual > 0 ? tq : n_tokens;
    const int v0 = ns;  // first quantized value token (S, or n_tokens while n_tokens < S)
    const int vbx = vq > v0 ? value_blocks(vq - v0, p.D) : 0;
    const size_t vblocks = (size_t)vbx * nbh;
    const T* vsrc = v + (size_t)v0 * p.D;  // token v0 of sequence/head 0; rows of n_tokens
    const int gpb = key_groups_per_block<T>(p.D);
    const int kgx = g_end > g_begin ? (g_end - g_begin + gpb - 1) / gpb : 0;
    const size_t kblocks = (size_t)kgx * nbh;
    bool values_done = false;
    if (kblocks > 0 && vblocks > 0 && kblocks + vblocks <= (size_t)UINT32_MAX) {
        // both codecs in one launch
        if (p.D == 128)
            launch_kv_d<T, 128>(p, k, n_tokens, g_begin, g_end, kgx, (unsigned)kblocks, vsrc,
                                vq - v0, v0, vbx, (unsigned)vblocks, stream);
        else
            launch_kv_d<T, 64>(p, k, n_tokens, g_begin, g_end, kgx, (unsigned)kblocks, vsrc,
                               vq - v0, v0, vbx, (unsigned)vblocks, stream);
        values_done = true;
    } else if (kblocks > 0) {
        quantize_channel_groups<T>(p, p.k_codes, p.k_meta, p.kbits, k, n_tokens, g_begin, g_end,
                                   stream);
    }
    auto copy = [&](const T* src, void* dst, int slots, int t0, int t1) {
        const size_t total = (size_t)nbh * (t1 - t0) * p.D;
        if (total > 0)
            copy_tail_kernel<T><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
                p, src, static_cast<T*>(dst), slots, n_tokens, t0, t1, total);
    };
    copy(k, p.k_tail, p.ring, tq, n_tokens);
    copy(k, p.k_sink, p.sink, 0, ns);
    copy(v, p.v_sink, p.sink, 0, ns);
    if (p.residual > 0)
        copy(v, p.v_tail, p.ring, tq, n_tokens);
    if (vblocks > 0 && !values_done)
        launch_token_groups<T>(p, p.vbits, vsrc, vq - v0, n_tokens, v0, stream);
    return hipGetLastError();
}

template <typename T, int KBITS, int VBITS>
void append_geometry(const Planes& p, const T* k, const T* v, int n, hipStream_t stream)
{
    const int nbh = p.nb * p.hkv;
    switch (p.geometry) {
    case 1: append_geometry_kernel<T, KBITS, VBITS, 1><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    case 2: append_geometry_kernel<T, KBITS, VBITS, 2><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    case 3: append_geometry_kernel<T, KBITS, VBITS, 3><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    }
}

template <typename T, int KBITS>
void append_kb(const Planes& p, const T* k, const T* v, int n, hipStream_t stream)
{
    const int nbh = p.nb * p.hkv;
    if (p.geometry != 0) {
        switch (p.vbits) {
        case 2: append_geometry<T, KBITS, 2>(p, k, v, n, stream); break;
        case 4: append_geometry<T, KBITS, 4>(p, k, v, n, stream); break;
        case 8: append_geometry<T, KBITS, 8>(p, k, v, n, stream); break;
        }
        return;
    }
    if (p.residual > 0) {
        switch (p.vbits) {
        case 2: append_residual_kernel<T, KBITS, 2><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
        case 4: append_residual_kernel<T, KBITS, 4><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
        case 8: append_residual_kernel<T, KBITS, 8><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
        }
        return;
    }
    switch (p.vbits) {
    case 2: append_kernel<T, KBITS, 2><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    case 4: append_kernel<T, KBITS, 4><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    case 8: append_kernel<T, KBITS, 8><<<nbh, p.D, 0, stream>>>(p, k, v, n); break;
    }
}

template <typename T>
hipError_t append_t(const Planes& p, const T* k, const T* v, int n, hipStream_t stream)
{
    switch (p.kbits) {
    case 2: append_kb<T, 2>(p, k, v, n, stream); break;
    case 4: append_kb<T, 4>(p, k, v, n, stream); break;
    case 8: append_kb<T, 8>(p, k, v, n, stream); break;
    }
    return hipGetLastError();
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

}  // namespace kvqi
