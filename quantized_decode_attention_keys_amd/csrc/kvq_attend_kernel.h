// kvq_attend_kernel.h -- fused decode attention over the quantized cache for
// gfx950: unpack -> dequantize -> rotary embedding -> q.k -> online softmax
// -> weighted sum of values.  When the token range of a (sequence, KV head)
// is split over several blocks, a small second kernel merges their partials.
//
// Method (web pages): keys are stored per channel over G-token groups and
// rotated after dequantization ("Your KV Cache Doesn't Have a Bit
// Problem...", sections "Keys: The Outliers Live in Fixed Channels" and
// "Rotary Embeddings Complicate the Keys"); the output is the softmax-weighted
// sum of the per-token-quantized value vectors (section "Values: Where the
// Intuition Breaks"); the whole cache is read for every generated token
// (section "Why the KV Cache Is Where This Bites").
//
// Work decomposition.  Grid = (splits, batch * kv_heads), W waves per block
// (W from the launch).  Each wave takes whole key groups in turn (waves never
// wait on each other inside the loop), keeps its own online-softmax state,
// and prefetches the next group's key and value words while it computes the
// current one (in the one-head head_dim-128 variants with 2-bit values the
// values lag one step: a step scores its group and adds the previous
// group's values).  The block merges its waves at the end; with one split it
// writes the output, otherwise (o, m, l) partials for the combine kernel.
//
// Key side, one group of 32 tokens: lane = channel pair i (64 pairs for
// head_dim 128; for head_dim 64 a wave takes two groups, 32 lanes each).
// Writing q' for the rotated query and (x, y) = (z0 + s0 c0, z1 + s1 c1) for
// the dequantized pair of token t = gG + j, the pair's score term is
//   Re[ conj(q'_i) e^{i t theta_i} (x + i y) ]
//     = Re[ T_j (Q_g (x + i y)) ],  T_j = e^{i j theta_i},  Q_g = conj(q'_i) e^{i gG theta_i},
// so per (group, pair) six constants fold dequantization and the group
// rotation, and per token the lane spends 4 FMAs on Q_g (x + i y) and 2 on
// the per-token twiddle T_j, staged once per block in LDS.  The per-pair
// partial scores of a token are summed across lanes through LDS, or, with
// one query head, head_dim 128 and 2-bit keys, by DPP row rotations read by
// the twiddle FMAs themselves and two cross-row swaps (see row_dpp_scores).
//
// Code unpacking.  A B-bit field masked in place inside a 16-bit half of a
// code word, with its lowest bit at position e <= 9, is the binary16 bit
// pattern of the subnormal c * 2^(e-24): exact, and read directly as an fp16
// operand by v_fma_mix_f32.  Fields that would reach the exponent bits are
// first shifted down.  The power of two 2^(e-24) is folded into the
// per-token twiddle (keys) or into one rescale at the end (values), so a
// 32-bit word of codes costs one AND per two codes plus one shift.
//
// Value side: the per-token weight p_t * step multiplies the codes and
// p_t * zero is accumulated once per (token, channel group).  With head_dim
// 128 a lane takes whole channel groups of two (or four) tokens, and
// v_dot2_f32_f16 adds the products of two tokens at once: the weights as a
// binary16 pair, the two tokens' codes of a channel as the same field of
// one word (see softmax_values).  With head_dim 64 a lane takes one 32-bit
// code word of a token row (32/B channels) per token slot.
#pragma once

#include "kvq_append.h"
#include "kvq_internal.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace kvqi {
namespace {

constexpr int G = kGroup;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxWaves = 16;  // max_block_waves over all variants

// Group scheduling.  With several query heads per KV head, groups after
// each wave's first are taken from a block counter as waves become ready
// (same-box A/B, GQA: 543 -> 521 us per step), and the wave priorities are
// left alone; the sums then run in an order that varies between calls, so
// results vary by fp32 rounding.  With one query head, waves take static
// shares paced by their priorities (the counter measured no faster on the
// 7B workload and 1.5 % slower on the 13B one), and results are
// reproducible.
constexpr bool dynamic_groups(int qpk) { return qpk > 1; }

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// Element idx of an fp16 (dtype 0) or fp32 (dtype 1) array.
__device__ __forceinline__ float ldf(const void* base, size_t idx, int dtype)
{
    return dtype == 0 ? __half2float(static_cast<const __half*>(base)[idx])
                      : static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// N consecutive 32-bit words (N a multiple of 4, 16-byte aligned address).
template <int N>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ src, uint32_t (&w)[N])
{
    static_assert(N % 4 == 0, "vector loads of 4 words");
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const uint4 v = reinterpret_cast<const uint4*>(src)[k];
        w[4 * k] = v.x;
        w[4 * k + 1] = v.y;
        w[4 * k + 2] = v.z;
        w[4 * k + 3] = v.w;
    }
}

// Layout of B-bit codes inside one 32-bit word: the low 16-bit half holds
// fields 0..TPH-1, the high half the next TPH; field f of a half sits at bits
// [f*B, f*B + B).  Fields f < DIRECT lie inside the fp16 mantissa (bits
// 0..9) and are masked in place; the others are read after a right shift by
// SHIFT bits.
template <int B>
struct Codec {
    static constexpr int TPH = 16 / B;        // fields per 16-bit half
    static constexpr int DIRECT = 10 / B;     // fields readable in place
    static constexpr int SHIFT = DIRECT * B;
    static constexpr uint32_t M2 = ((1u << B) - 1u) | (((1u << B) - 1u) << 16);
    // bit position of field f (as read) inside its half
    static constexpr int pos(int f) { return f < DIRECT ? f * B : (f - DIRECT) * B; }
    // distinct positions: 0, B, ..., (DIRECT-1)*B
    static constexpr int NSCALE = DIRECT;
    // field f of both halves, masked, as a pair of binary16 subnormals
    __device__ static __forceinline__ uint32_t field(uint32_t w, uint32_t w_shifted, int f)
    {
        return (f < DIRECT ? w : w_shifted) & (M2 << pos(f));
    }
};

__device__ __forceinline__ float lo_h(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v & 0xffffu))); }
__device__ __forceinline__ float hi_h(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v >> 16))); }

// Two binary16 values as one operand of v_dot2_f32_f16.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half2v pack_h2(float lo, float hi)
{
    half2v r;
    r.x = (_Float16)lo;  // nearest-even
    r.y = (_Float16)hi;
    return r;
}

// Operands of v_mfma_f32_16x16x32_f16: eight binary16 values per lane.
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// (a, b) as two binary16 pairs hi + lo: hi rounded toward zero, lo the
// remainder (exact in fp32) rounded toward zero, so a = hi.x + lo.x within
// 2^-20 |a| or 2^-24, whichever is larger (b likewise).  Products of such
// splits summed as hi*hi + hi*lo + lo*hi carry fp32-class accuracy through
// a binary16 matrix instruction (lo*lo, below 2^-20 of the product, is left
// out).  m1 is -1.0 held where the compiler cannot see its value: the
// remainders a - hi.x = hi.x * m1 + a then stay one v_fma_mix_f32 each,
// reading the binary16 half in place (a - hi.x would convert, then
// subtract).
__device__ __forceinline__ uint2 split_h2(float a, float b, float m1)
{
    const auto hi = __builtin_amdgcn_cvt_pkrtz(a, b);
    const float ra = fmaf((float)hi[0], m1, a), rb = fmaf((float)hi[1], m1, b);
    return make_uint2(__builtin_bit_cast(uint32_t, hi),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(ra, rb)));
}

// Value of v in another lane of the same 16-lane row (DPP, VALU only).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane k <-> 7-k within each 8
constexpr int kDppMirror = 0x140;     // lane k <-> 15-k within each 16
constexpr int kDppRor8 = 0x128;       // lane k <- lane (k+8) mod 16 within each 16

// As dpp<CTRL> for patterns that read a lane of the same row for every lane
// (quad permutations, mirrors), so no old value is needed.
template <int CTRL>
__device__ __forceinline__ float dpp_all(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// acc0 += x0(lane q - D) * t0 + y0(lane q - D) * u0 and the same for acc1,
// where x(lane q - D) is x in lane (q - D) mod 16 of the same 16-lane row
// (DPP row rotation, read by the FMA itself).  The s_nop gives the two wait
// states a DPP read needs after the VALU write of its source.
template <int D>
__device__ __forceinline__ void fmac_row_ror(float& acc0, float& acc1, float x0, float y0,
                                             float x1, float y1, float4 t)
{
    static_assert(D >= 1 && D <= 15, "row rotation");
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %2, %6 row_ror:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %7 row_ror:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %8 row_ror:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_ror:%10 row_mask:0xf bank_mask:0xf"
        : "+v"(acc0), "+v"(acc1)
        : "v"(x0), "v"(y0), "v"(x1), "v"(y1), "v"(t.x), "v"(t.y), "v"(t.z), "v"(t.w), "i"(D));
}

// Partial-score terms (x0, y0, x1, y1) of N positions of the two 16-token
// units of a lane's key words.
template <int N>
struct Terms {
    float4 v[N];
};

// f(std::integral_constant<int, k>) for k = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void for_each_int(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        for_each_int<B + 1, E>(f);
    }
}

// max(a, b) for operands that are never NaN: a compare and a select, where
// fmaxf would first quiet both operands.
__device__ __forceinline__ float max_nn(float a, float b) { return a > b ? a : b; }

// Cross-row exchanges on the VALU (no LDS round trip).  With both operands
// equal to v, the 16-lane swap returns {rows (0,0,2,2) of v, rows (1,1,3,3)}
// and the 32-lane swap {lanes 0..31 of v twice, lanes 32..63 twice}.
struct Pair {
    float a, b;
};
__device__ __forceinline__ Pair swap16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ Pair swap32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// v[l] + v[l ^ 32], the same bits in both lanes.
__device__ __forceinline__ float half_sum(float v)
{
    const Pair r = swap32(v);
    return r.a + r.b;
}

// Maximum over the wave: four DPP steps inside each 16-lane row, then the
// cross-row swaps.  HALVES_EQUAL: lanes l and l + 32 hold the same value, so
// the 32-lane step is skipped.
template <bool HALVES_EQUAL>
__device__ __forceinline__ float wave_max(float v)
{
    v = max_nn(v, dpp_all<kDppXor1>(v));
    v = max_nn(v, dpp_all<kDppXor2>(v));
    v = max_nn(v, dpp_all<kDppHalfMirror>(v));
    v = max_nn(v, dpp_all<kDppMirror>(v));
    const Pair r = swap16(v);
    v = max_nn(r.a, r.b);
    if (!HALVES_EQUAL) {
        const Pair t = swap32(v);
        v = max_nn(t.a, t.b);
    }
    return v;
}

// Sum over the wave (the same value in every lane, up to the order of the
// additions): as wave_max.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    const Pair r = swap16(v);
    v = r.a + r.b;
    const Pair t = swap32(v);
    return t.a + t.b;
}

template <int D, int KB, int VB, int QPK>
struct Shape {
    static constexpr int NP = D / 2;           // channel pairs
    static constexpr int GPW = 64 / NP;        // key groups per wave step
    static constexpr int TPW = G * GPW;        // tokens per wave step
    static constexpr int WK = KB;              // words per (key group, channel)
    static constexpr int WV = VB;              // words per (token, value group)
    static constexpr int NCG = D / G;          // value groups per token
    static constexpr int WPT = NCG * WV;       // value code words per token
    static constexpr int TS = 64 / WPT;        // token slots in the value phase
    static constexpr int VTOK = TPW / TS;      // value tokens per lane per step
    static constexpr int NC = 32 / VB;         // channels per value word
    static constexpr int RED_STRIDE = 33;      // floats per lane row of the reduce buffer
    static_assert(64 % WPT == 0 && TPW % TS == 0, "value lane mapping");
    // Value lane mapping.  Token pairs (one query head, head_dim 128): lane =
    // (row r = lane / 16, column c = lane % 16) takes tokens c and c + 16 of
    // the step and all 32 channels of value group r, so the weights it needs
    // sit in its own 16-lane row pair and one swap fetches both.  Otherwise
    // lane = (code word, token slot) as described at the top.
    // Token quads (several query heads, head_dim 128): lane (r, c) takes
    // tokens c, c^8, c+16 and (c^8)+16 of the step and code words
    // (2r + c/8) * NW .. + NW-1 of each (16 channels of one value group);
    // its weights come from one swap and two DPP row rotations.
    static constexpr bool PAIRS = (QPK == 1 && NP == 64);
    static constexpr bool QUADS = (QPK > 1 && NP == 64);
    static_assert(!(PAIRS || QUADS) || NCG == 4, "value groups per 16-lane row");
    static constexpr int NW = WPT / 8;                  // quads: words per (lane, token)
    static constexpr int NVW = PAIRS ? 2 * WV : QUADS ? 4 * NW : VTOK;  // value code words per lane per step
    static constexpr int NVM = PAIRS ? 2 : QUADS ? 4 : VTOK;            // value meta words per lane per step
    static constexpr int NCL = PAIRS ? G : QUADS ? NW * NC : NC;        // value channels per lane
    // One query head, head_dim 128, 2-bit keys (or 4-bit keys with 2-bit
    // values): a token's 64 partial scores are summed on the VALU (DPP row
    // rotations fused into the twiddle FMAs, then two cross-row swaps)
    // instead of through LDS; no reduce buffers.  (With 4-bit keys and
    // 4-bit values the rotations cost most of the saving and the main loop
    // spilled registers.)
    static constexpr bool ROWDPP = row_dpp_sums(D, KB, VB, QPK);
    static_assert(!ROWDPP || PAIRS, "row-DPP sums use the one-head value layout");
    static constexpr int WPU = KB / 2;          // row-DPP: key words per 16-token unit
    static constexpr int NRED = ROWDPP ? 0 : (QPK == 2 || QPK == 4) ? 2 : 1;  // reduce buffers per wave (heads alternate)
};

// Everything one wave step reads from memory, loaded one step ahead.
template <int WK, int NVW, int NVM>
struct StepData {
    uint32_t kw[2 * WK];   // key codes of the lane's two channels
    uint2 km;              // their (step, zero) meta words
    float2 rg;             // e^{i g G theta_i}
    uint32_t vw[NVW];      // value code words of the lane's value tokens
    uint32_t vm[NVM];      // their value meta words
};

// Per-wave online-softmax state and value accumulators.
template <int QPK, int NC>
struct WaveState {
    float m[QPK];      // running max (base-2 logits), uniform across the wave
    float l[QPK];      // this lane's share of the running sum
    float z[QPK];      // sum_t p_t * zero_{t, group of this lane's word}
    float o[QPK][NC];  // sum_t p_t * step * code * 2^(pos-24) per channel of the word
};

// Plane pointers of one (sequence, KV head); every index below them fits in
// 32 bits (the host caps max_tokens), so loads use a scalar base plus a
// 32-bit lane offset.
struct HeadPlanes {
    const uint32_t* kc;   // [gcap][D][WK]
    const uint32_t* km;   // [gcap][D]
    const uint32_t* vc;   // [tcap][WPT]
    const uint32_t* vm;   // [tcap][NCG]
};

// Value words of the lane's tokens among t0 .. t0 + TPW - 1.  Addresses are
// a wave-uniform base (scalar registers) plus a 32-bit lane offset.  CLAMP:
// some of those tokens may lie past t_last, the last token the cache holds;
// their indexes are clamped to it (the words are loaded but weigh 0).
template <int D, int KB, int VB, int QPK, bool CLAMP>
__device__ __forceinline__ void load_values(const HeadPlanes& hp, int lane, int t0, int t_last,
                                            uint32_t (&vw)[Shape<D, KB, VB, QPK>::NVW],
                                            uint32_t (&vm)[Shape<D, KB, VB, QPK>::NVM])
{
    using S = Shape<D, KB, VB, QPK>;
    const uint32_t* vc0 = hp.vc + (size_t)t0 * S::WPT;
    const uint32_t* vm0 = hp.vm + (size_t)t0 * S::NCG;
    auto slot = [&](unsigned tt) {
        return CLAMP ? (unsigned)(min(t0 + (int)tt, t_last) - t0) : tt;
    };
    if constexpr (S::PAIRS) {
        const unsigned r = lane >> 4, c = lane & 15;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const unsigned tt = slot(c + 16 * k);
            const uint32_t* src = vc0 + tt * S::WPT + r * S::WV;
            if constexpr (S::WV == 2) {
                const uint2 w = *reinterpret_cast<const uint2*>(src);
                vw[2 * k] = w.x;
                vw[2 * k + 1] = w.y;
            } else {
                uint32_t w[S::WV];
                load_words<S::WV>(src, w);
#pragma unroll
                for (int u = 0; u < S::WV; ++u)
                    vw[k * S::WV + u] = w[u];
            }
            vm[k] = vm0[tt * S::NCG + r];
        }
    } else if constexpr (S::QUADS) {
        const unsigned r = lane >> 4, c = lane & 15;
        const unsigned w0 = (2 * r + (c >> 3)) * S::NW, vg = w0 / S::WV;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // slots 0..3: tokens c, c^8, c+16, (c^8)+16
            const unsigned tt = slot((k & 1 ? (c ^ 8u) : c) + (k & 2 ? 16u : 0u));
            const uint32_t* src = vc0 + tt * S::WPT + w0;
            if constexpr (S::NW == 1) {
                vw[k] = src[0];
            } else if constexpr (S::NW == 2) {
                const uint2 w = *reinterpret_cast<const uint2*>(src);
                vw[2 * k] = w.x;
                vw[2 * k + 1] = w.y;
            } else {
                uint32_t w[S::NW];
                load_words<S::NW>(src, w);
#pragma unroll
                for (int u = 0; u < S::NW; ++u)
                    vw[k * S::NW + u] = w[u];
            }
            vm[k] = vm0[tt * S::NCG + vg];
        }
    } else {
        const unsigned w = lane % S::WPT, vslot = lane / S::WPT, vcg = w / S::WV;
#pragma unroll
        for (int k = 0; k < S::VTOK; ++k) {
            const unsigned tt = slot(vslot + k * S::TS);
            vw[k] = vc0[tt * S::WPT + w];
            vm[k] = vm0[tt * S::NCG + vcg];
        }
    }
}

// Key words, metadata and group rotation of key group gb (and gb + 1 for
// head_dim 64); gb <= g1 - 1.
template <int D, int KB, int VB, int QPK>
__device__ __forceinline__ void load_keys(
    const HeadPlanes& hp, const float2* __restrict__ rope_group, int lane, int gb, int g1,
    StepData<KB, Shape<D, KB, VB, QPK>::NVW, Shape<D, KB, VB, QPK>::NVM>& sd)
{
    using S = Shape<D, KB, VB, QPK>;
    const unsigned i = lane % S::NP, gsub = lane / S::NP;
    // head_dim 64: the second group of the step, if any, else the first again
    const unsigned gl = (S::GPW > 1 && gsub != 0 && gb + 1 < g1) ? 1u : 0u;
    const unsigned ci = gl * D + 2 * i;
    load_words<2 * S::WK>(hp.kc + (size_t)gb * (D * S::WK) + ci * S::WK, sd.kw);
    sd.km = *reinterpret_cast<const uint2*>(hp.km + (size_t)gb * D + ci);
    sd.rg = rope_group[(size_t)gb * S::NP + gl * S::NP + i];
}

// Whether a step tests for a raised maximum before the wave reduction and
// rescale (a ballot), rather than always doing both.  Measured faster with
// 2-bit values or several query heads, slower with one head and 4-bit values.
constexpr bool skips_rescale(int vb, int qpk) { return qpk > 1 || vb <= 2; }

// Online-softmax update for one wave step.  Lane `lane` holds score s[h] of
// token tt = lane (head_dim 64) or lane & 31 (head_dim 128), i.e. token
// t_base + tt; tokens at or past t_end are absent and weigh exactly 0.
// Returns in pw[h] the weight of the lane's own token.
template <int D, int KB, int VB, int QPK>
__device__ __forceinline__ void softmax_weights(int lane, int t_base, int t_end,
                                                const float (&s)[QPK], float (&pw)[QPK],
                                                WaveState<QPK, Shape<D, KB, VB, QPK>::NCL>& st)
{
    using S = Shape<D, KB, VB, QPK>;
    const int tt_own = (S::NP == 64) ? (lane & 31) : lane;
    const bool own_valid = t_base + tt_own < t_end;
    const bool counts = (S::NP == 32) || lane < 32;  // head_dim 128: lanes l, l+32 share a token
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
        const float sv = own_valid ? s[h] : -INFINITY;
        // Most steps raise no score above the running maximum (one compare
        // and a ballot tell); with skips_rescale only the others reduce the
        // wave's maximum and rescale.  Either way m_new = max(m, scores), bit
        // for bit.
        const bool raises = !skips_rescale(VB, QPK) ||
                            __builtin_amdgcn_ballot_w64(sv > st.m[h]) != 0;  // uniform
        if (raises) {
            const float m_new = max_nn(st.m[h], wave_max<S::NP == 64>(sv));
            // arguments <= 0; v_exp_f32 returns 0 for -inf and for results
            // below the fp32 normal range, which weigh nothing at this
            // tolerance
            const float alpha = __builtin_amdgcn_exp2f(st.m[h] - m_new);  // 0 on the first step
            st.l[h] *= alpha;
            st.m[h] = m_new;
            if (alpha != 1.f) {  // uniform across the wave
                st.z[h] *= alpha;
#pragma unroll
                for (int c = 0; c < S::NCL; ++c)
                    st.o[h][c] *= alpha;
            }
        }
        const float pl = own_valid ? __builtin_amdgcn_exp2f(sv - st.m[h]) : 0.f;
        st.l[h] += counts ? pl : 0.f;
        pw[h] = pl;
    }
}

// Accumulation of one wave step's value tokens from their code words with
// their softmax weights pw (absent tokens weigh 0, whatever their words).
template <int D, int KB, int VB, int QPK>
__device__ __forceinline__ void accumulate_values(int lane, const float (&pw)[QPK],
                                                  const uint32_t* vwords, const uint32_t* vmetas,
                                                  WaveState<QPK, Shape<D, KB, VB, QPK>::NCL>& st)
{
    using S = Shape<D, KB, VB, QPK>;
    using C = Codec<VB>;
    if constexpr (S::PAIRS) {
        // weights of tokens c and c + 16: lanes of rows 0 and 2 hold token
        // c's, rows 1 and 3 token c + 16's
        const Pair pp = swap16(pw[0]);  // 0 for absent tokens
        st.z[0] = fmaf(pp.a, hi_h(vmetas[0]), st.z[0]);
        st.z[0] = fmaf(pp.b, hi_h(vmetas[1]), st.z[0]);
        // One dot2 takes a channel of both tokens: the weights p * step as
        // a binary16 pair (token c low, c + 16 high), the codes as the same
        // field of the two tokens' half-words brought into one word.
        const half2v w2 = pack_h2(pp.a * lo_h(vmetas[0]), pp.b * lo_h(vmetas[1]));
#pragma unroll
        for (int u = 0; u < S::WV; ++u) {
            const uint32_t wa = vwords[u], wb = vwords[S::WV + u];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // half hh of each token's word: channels hh * TPH .. of word u
                const uint32_t word = __builtin_amdgcn_perm(wb, wa, hh ? 0x07060302u : 0x05040100u);
                const uint32_t wsh = word >> C::SHIFT;
#pragma unroll
                for (int f = 0; f < C::TPH; ++f) {
                    const int cc = u * S::NC + hh * C::TPH + f;
                    st.o[0][cc] = __builtin_amdgcn_fdot2(
                        w2, __builtin_bit_cast(half2v, C::field(word, wsh, f)), st.o[0][cc], false);
                }
            }
        }
        return;
    }
    if constexpr (S::QUADS) {
        // Token slots k = 0..3 are tokens c, c^8, c+16, (c^8)+16; slots k and
        // k + 2 go through v_dot2_f32_f16 together, as in the one-head
        // variant: their half-words brought into one word by one perm (shared
        // by every head), their weights p * step as one binary16 pair.
        half2v w2[QPK][2];
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            // tokens c and c + 16 from the row pair, c^8 and (c^8) + 16 by
            // rotating those by 8 lanes inside the row
            const Pair pp = swap16(pw[h]);
            const float pk[4] = {pp.a, dpp<kDppRor8>(pp.a), pp.b, dpp<kDppRor8>(pp.b)};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                st.z[h] = fmaf(pk[k], hi_h(vmetas[k]), st.z[h]);  // 0 for absent tokens
#pragma unroll
            for (int k = 0; k < 2; ++k)
                w2[h][k] = pack_h2(pk[k] * lo_h(vmetas[k]), pk[k + 2] * lo_h(vmetas[k + 2]));
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
            for (int u = 0; u < S::NW; ++u) {
                const uint32_t wa = vwords[k * S::NW + u], wb = vwords[(k + 2) * S::NW + u];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t word =
                        __builtin_amdgcn_perm(wb, wa, hh ? 0x07060302u : 0x05040100u);
                    const uint32_t wsh = word >> C::SHIFT;
#pragma unroll
                    for (int f = 0; f < C::TPH; ++f) {
                        const half2v m = __builtin_bit_cast(half2v, C::field(word, wsh, f));
                        const int cc = u * S::NC + hh * C::TPH + f;
#pragma unroll
                        for (int h = 0; h < QPK; ++h)
                            st.o[h][cc] = __builtin_amdgcn_fdot2(w2[h][k], m, st.o[h][cc], false);
                    }
                }
            }
        }
        return;
    }
    const int vslot = lane / S::WPT;
#pragma unroll
    for (int k = 0; k < S::VTOK; ++k) {
        const int tt = vslot + k * S::TS;
        const uint32_t word = vwords[k];
        const uint32_t wsh = word >> C::SHIFT;
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const float pt = __shfl(pw[h], tt);  // 0 for absent tokens
            const float ps = pt * lo_h(vmetas[k]);
            st.z[h] = fmaf(pt, hi_h(vmetas[k]), st.z[h]);
#pragma unroll
            for (int f = 0; f < C::TPH; ++f) {
                const uint32_t m = C::field(word, wsh, f);
                st.o[h][f] = fmaf(ps, lo_h(m), st.o[h][f]);
                st.o[h][C::TPH + f] = fmaf(ps, hi_h(m), st.o[h][C::TPH + f]);
            }
        }
    }
}

// Softmax update for one wave step and accumulation of its value tokens.
template <int D, int KB, int VB, int QPK>
__device__ __forceinline__ void softmax_values(int lane, int t_base, int t_end,
                                               const float (&s)[QPK], const uint32_t* vwords,
                                               const uint32_t* vmetas,
                                               WaveState<QPK, Shape<D, KB, VB, QPK>::NCL>& st)
{
    float pw[QPK];
    softmax_weights<D, KB, VB, QPK>(lane, t_base, t_end, s, pw, st);
    accumulate_values<D, KB, VB, QPK>(lane, pw, vwords, vmetas, st);
}

// N consecutive elements of an fp16 (dtype 0) or fp32 row as floats; N a
// multiple of 4, the address 8-byte (fp16, N = 4) or 16-byte aligned.
template <int N>
__device__ __forceinline__ void load_row(const void* src, int dtype, float (&x)[N])
{
    if (dtype == 0) {
        const uint32_t* w = static_cast<const uint32_t*>(src);
        uint32_t u[N / 2];
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int k = 0; k < N / 8; ++k) {
                const uint4 v = reinterpret_cast<const uint4*>(w)[k];
                u[4 * k] = v.x;
                u[4 * k + 1] = v.y;
                u[4 * k + 2] = v.z;
                u[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < N / 4; ++k) {
                const uint2 v = reinterpret_cast<const uint2*>(w)[k];
                u[2 * k] = v.x;
                u[2 * k + 1] = v.y;
            }
        }
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            x[2 * k] = lo_h(u[k]);
            x[2 * k + 1] = hi_h(u[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const float4 v = static_cast<const float4*>(src)[k];
            x[4 * k] = v.x;
            x[4 * k + 1] = v.y;
            x[4 * k + 2] = v.z;
            x[4 * k + 3] = v.w;
        }
    }
}

// Softmax update for one wave step of unquantized values (the residual
// window): rows[tt] is token t_base + tt's value row (rows of D elements,
// tokens 0 .. cnt-1 present).  Each lane covers the same (token, channel)
// pairs as for code words, and adds p * v * 2^(pos-24) to the accumulator
// of a code at bit position pos of that channel, so the one final rescale by
// 2^(24-pos) serves both.
template <int D, int KB, int VB, int QPK>
__device__ __forceinline__ void softmax_fp_values(int lane, int t_base, int cnt,
                                                  const float (&s)[QPK], const void* rows,
                                                  int dtype,
                                                  WaveState<QPK, Shape<D, KB, VB, QPK>::NCL>& st)
{
    using S = Shape<D, KB, VB, QPK>;
    using C = Codec<VB>;
    float pw[QPK];
    softmax_weights<D, KB, VB, QPK>(lane, t_base, t_base + cnt, s, pw, st);
    const size_t esz = dtype == 0 ? 2 : 4;
    auto row = [&](int tt, int ch) {  // absent tokens read the last present row
        return static_cast<const char*>(rows) + ((size_t)min(tt, cnt - 1) * D + ch) * esz;
    };
    auto scale = [](int cc) { return 1.0f / (float)(1 << (24 - C::pos(cc % C::TPH))); };
    if constexpr (S::PAIRS) {
        const Pair pp = swap16(pw[0]);
        const int r = lane >> 4, c = lane & 15;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float pt = k ? pp.b : pp.a;
            float x[G];
            load_row<G>(row(c + 16 * k, r * G), dtype, x);
#pragma unroll
            for (int cc = 0; cc < G; ++cc)
                st.o[0][cc] = fmaf(pt * scale(cc), x[cc], st.o[0][cc]);
        }
    } else if constexpr (S::QUADS) {
        const int r = lane >> 4, c = lane & 15;
        const int ch0 = (2 * r + (c >> 3)) * S::NW * S::NC;
        float pk[QPK][4];
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const Pair pp = swap16(pw[h]);
            pk[h][0] = pp.a;
            pk[h][1] = dpp<kDppRor8>(pp.a);
            pk[h][2] = pp.b;
            pk[h][3] = dpp<kDppRor8>(pp.b);
        }
        // one token row at a time, added into every head
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            constexpr int NCH = S::NW * S::NC;  // 16 channels
            float x[NCH];
            load_row<NCH>(row((k & 1 ? (c ^ 8) : c) + (k & 2 ? 16 : 0), ch0), dtype, x);
#pragma unroll
            for (int h = 0; h < QPK; ++h)
#pragma unroll
                for (int cc = 0; cc < NCH; ++cc)
                    st.o[h][cc] = fmaf(pk[h][k] * scale(cc), x[cc], st.o[h][cc]);
        }
    } else {
        const int w = lane % S::WPT, vslot = lane / S::WPT;
#pragma unroll
        for (int k = 0; k < S::VTOK; ++k) {
            const int tt = vslot + k * S::TS;
            float x[S::NC];
            load_row<S::NC>(row(tt, w * S::NC), dtype, x);
#pragma unroll
            for (int h = 0; h < QPK; ++h) {
                const float pt = __shfl(pw[h], tt);
#pragma unroll
                for (int cc = 0; cc < S::NC; ++cc)
                    st.o[h][cc] = fmaf(pt * scale(cc), x[cc], st.o[h][cc]);
            }
        }
    }
}

// Variants whose values lag their keys by one step (the one-head head_dim-128
// variants with 2-bit values): deferring the others' values spilled registers
// (GQA 589 -> 870 us, 13B at 4/4 bits 178 -> 185 us; 7B 37.5 -> 36.9 us).
constexpr bool defers_values(int kb, int vb, int qpk, int np)
{
    return qpk == 1 && vb == 2 && np == 64 && kb <= 8;
}

// Variants whose unquantized chunks are scored before their groups: those
// that compile without extra register spills that way (the others score
// them after their groups).
constexpr bool chunks_first(int kb, int vb, int qpk) { return qpk == 1 && vb == 2 && kb <= 4; }

template <int D, int KB, int VB, int QPK>
__global__ __launch_bounds__(64 * max_block_waves(QPK)) void attend_kernel(Planes p, const void* __restrict__ q,
                                                                float* __restrict__ out, int n,
                                                                int splits, int hgroups,
                                                                const void* __restrict__ k_new,
                                                                const void* __restrict__ v_new)
{
    using S = Shape<D, KB, VB, QPK>;
    using KC = Codec<KB>;
    using VC = Codec<VB>;
    constexpr int NP = S::NP;
    constexpr int RS = S::RED_STRIDE;
    // [nwaves][64][RS] reduce buffers, reused for the merge; 16-byte aligned
    // for the 16-byte operand reads of the matrix-core scores
    extern __shared__ __attribute__((aligned(16))) float smem[];

    const int nwaves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
    const int i = lane % NP, gsub = lane / NP;
    const int split = blockIdx.x;
    // block y = (sequence, KV head, group of QPK of its query heads)
    const size_t bh = blockIdx.y / hgroups;
    const int b = (int)(bh / p.hkv), kvh = (int)(bh % p.hkv);
    const int head0 = (kvh * hgroups + (int)(blockIdx.y % hgroups)) * QPK;
    // Tokens [0, ns) are in the sinks, groups [gs, gs + ngq) quantized, and
    // tokens [tq, n) in the tail rings (keys always, values with a residual
    // window); sink and ring tokens go in chunks of G taken by the waves of
    // the last split.
    const int ns = n < p.sink ? n : p.sink;
    const int tq = quantized_end(n, p.residual, p.sink), gs = p.sink / G;
    const int ngq = tq / G > gs ? tq / G - gs : 0;
    const int nsink_chunks = (ns + G - 1) / G;
    const int nchunks = nsink_chunks + (n - tq + G - 1) / G;
    const int g0 = gs + (int)((long long)split * ngq / splits);
    const int g1 = gs + (int)((long long)(split + 1) * ngq / splits);

    // Decode step in one launch (k_new != null; plain cache, one block per
    // (sequence, KV head) and split): the last split's block first appends
    // token n-1 -- its value quantized per token, its key into the tail and,
    // when it completes group (n-1)/G, that group quantized.  Everything the
    // append writes is read only by this block, and only after the barrier
    // below (every load of cache words comes after it).
    const bool appends = k_new != nullptr && split == splits - 1;

    HeadPlanes hp;
    hp.kc = p.k_codes + bh * (size_t)p.gcap * D * S::WK;
    hp.km = p.k_meta + bh * (size_t)p.gcap * D;
    hp.vc = p.v_codes + bh * (size_t)p.tcap * S::WPT;
    hp.vm = p.v_meta + bh * (size_t)p.tcap * S::NCG;
    const int stride = nwaves * S::GPW;
    constexpr bool kDynamicGroups = dynamic_groups(QPK);
    // Several query heads and head_dim 128: the heads' scores on the matrix
    // cores (one lane per channel pair, a whole group per wave step).
    constexpr bool kMfmaHeads = QPK > 1 && NP == 64;
    constexpr int kUS = 64;  // words per row of the MFMA operand staging
    static_assert(!kMfmaHeads || (32 + 2 * QPK) * kUS <= S::NRED * 64 * RS,
                  "operand staging inside the wave's reduce buffers");
    StepData<KB, S::NVW, S::NVM> cur, nxt;
    int gb = g0 + wave * S::GPW;
    if (appends && threadIdx.x < D) {  // whole waves: D is a multiple of 64
        const int c = threadIdx.x;
        const int t = n - 1;
        if (p.dtype == 0) {
            const __half* kn = static_cast<const __half*>(k_new) + bh * D;
            const __half* vn = static_cast<const __half*>(v_new) + bh * D;
            append_token_groups<__half, VB>(p.v_codes, p.v_meta, p.tcap, vn, bh, t, c, D);
            append_channel_groups<__half, KB>(p.k_codes, p.k_meta, p.gcap,
                                              static_cast<__half*>(p.k_tail) + bh * p.ring * D,
                                              kn[c], bh, t, c, D);
        } else {
            const float* kn = static_cast<const float*>(k_new) + bh * D;
            const float* vn = static_cast<const float*>(v_new) + bh * D;
            append_token_groups<float, VB>(p.v_codes, p.v_meta, p.tcap, vn, bh, t, c, D);
            append_channel_groups<float, KB>(p.k_codes, p.k_meta, p.gcap,
                                             static_cast<float*>(p.k_tail) + bh * p.ring * D,
                                             kn[c], bh, t, c, D);
        }
    }

    // conj(q') * log2(e)/sqrt(D) for this lane's pair, q' = q rotated to n-1
    float2 qc[QPK];
    {
        const int pos = n - 1;
        const float2 rot = cmul(p.rope_group[(size_t)(pos / G) * NP + i],
                                p.rope_offset[(pos % G) * NP + i]);
        const float scale = kLog2e * rsqrtf((float)D);
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const size_t qi = ((size_t)(b * p.hq + head0 + h)) * D + 2 * i;
            const float2 qq = cmul(make_float2(ldf(q, qi, p.dtype), ldf(q, qi + 1, p.dtype)), rot);
            qc[h] = make_float2(qq.x * scale, -qq.y * scale);
        }
    }
    // Per-token twiddles e^{i j theta_i}, pre-scaled by 2^(24 - pos) of the
    // field that holds token j (j = word * 2*TPH + half * TPH + field), staged
    // once per block: entry (j/2, pair) holds tokens j and j+1 as
    // (T.x, -T.y) pairs.  A separate array from the reduce buffers, so its
    // reads are never ordered after their writes.
    // With the row-DPP sums (S::ROWDPP) the table is laid out for them
    // instead: entry (d, pair i), d = 0..15, holds for lane q = i % 16 of row
    // i / 16 the twiddles of the pair i' = row lane (q - d) mod 16 that the
    // DPP rotation by d brings in, for token q (.x, .y) and token 16 + q
    // (.z, .w), scaled by 2^(24 - pos) of word position d, where that pair's
    // lane keeps those tokens after its rotation by i' % 16 tokens.
    __shared__ float4 twl[G / 2 * 64];
    for (int idx = threadIdx.x; idx < G / 2 * NP; idx += blockDim.x) {
        if constexpr (S::ROWDPP) {
            const int d = idx / NP, ii = idx % NP, qq = ii & 15;
            const int ip = (ii & ~15) | ((qq - d) & 15);
            const float sc = (float)(1 << (24 - KC::pos(d % KC::TPH)));
            const float2 t0 = p.rope_offset[qq * NP + ip];
            const float2 t1 = p.rope_offset[(16 + qq) * NP + ip];
            twl[idx] = make_float4(t0.x * sc, -t0.y * sc, t1.x * sc, -t1.y * sc);
        } else {
            const int jp = idx / NP, ii = idx % NP;
            const float2 t0 = p.rope_offset[(2 * jp) * NP + ii];
            const float2 t1 = p.rope_offset[(2 * jp + 1) * NP + ii];
            const float sc0 = (float)(1 << (24 - KC::pos((2 * jp) % KC::TPH)));
            const float sc1 = (float)(1 << (24 - KC::pos((2 * jp + 1) % KC::TPH)));
            twl[idx] = make_float4(t0.x * sc0, -t0.y * sc0, t1.x * sc1, -t1.y * sc1);
        }
    }
    // Groups after each wave's first one are taken from a block counter as
    // waves become ready (LDS atomic by one lane), so a wave that also
    // scores unquantized chunks, or that its SIMD serves later, simply takes
    // fewer groups and the waves finish together.
    __shared__ int group_next;
    if (kDynamicGroups && threadIdx.x == 0)
        group_next = g0 + stride;
    __syncthreads();  // also orders the append's global writes before every read of them
    // Every wave reads the twiddles from LDS where it uses them: tw_base is
    // re-made opaque every step, so the compiler cannot hoist those reads
    // into 64 registers held for the whole loop.
    int tw_base = i;
    auto twiddle = [&](int j) {
        const float4 t = twl[(j >> 1) * NP + tw_base];
        return (j & 1) ? make_float2(t.z, t.w) : make_float2(t.x, t.y);
    };
    // Row-DPP sums: the two tokens of lane q (q and 16 + q) over the 64
    // pairs.  The key words of a channel form two 16-token units (tokens
    // 0..15 and 16..31; one word each at 2 bits, two at 4).  Every lane
    // rotates each unit by q tokens, so its position d (0..15) holds token
    // d + q mod 16 of the unit; then position d of the lane q - d of the
    // same row holds token q of the unit, and a DPP rotation by d brings it
    // in.  Each lane sums its two tokens over the 16 pairs of its row, and
    // two cross-row swaps finish the sums.  term(f) gives, for positions
    // p * TPH + f, p < NPOS (code field f of each half-word of a unit), the
    // (X, Y) = Q (x + iy) of unit 0 and of unit 1 at the field scale of that
    // position; the twiddle table (T.x, -T.y) * 2^(24 - pos) turns them into
    // partial scores.  Returns the score of token lane % 32 (the layout of
    // the LDS sums).
    constexpr int NPOS = 2 * S::WPU;
    auto row_dpp_scores = [&](auto&& term) __attribute__((always_inline)) {
        float acc0 = 0.f, acc1 = 0.f;
        for_each_int<0, KC::TPH>([&](auto ff) __attribute__((always_inline)) {
            constexpr int f = decltype(ff)::value;
            const Terms<NPOS> v = term(f);
            for_each_int<0, NPOS>([&](auto pp) __attribute__((always_inline)) {
                constexpr int pi = decltype(pp)::value, d = pi * KC::TPH + f;
                const float4 t = twl[d * NP + tw_base];
                if constexpr (d == 0) {  // the lane's own pair
                    acc0 = fmaf(t.x, v.v[pi].x, t.y * v.v[pi].y);
                    acc1 = fmaf(t.z, v.v[pi].z, t.w * v.v[pi].w);
                } else {
                    fmac_row_ror<d>(acc0, acc1, v.v[pi].x, v.v[pi].y, v.v[pi].z, v.v[pi].w, t);
                }
            });
        });
        auto rows = [](float v) {
            const Pair r = swap16(v);
            v = r.a + r.b;
            const Pair t = swap32(v);
            return t.a + t.b;
        };
        acc0 = rows(acc0);
        acc1 = rows(acc1);
        return (lane & 16) ? acc1 : acc0;
    };

    WaveState<QPK, S::NCL> st;
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.f;
        st.z[h] = 0.f;
#pragma unroll
        for (int c = 0; c < S::NCL; ++c)
            st.o[h][c] = 0.f;
    }
    float* red = smem + wave * S::NRED * 64 * RS;
    const int red_half = lane & ~31, red_col = lane & 31;

    // Waves of a SIMD otherwise run oldest-first, so the oldest finishes its
    // share long before the youngest, which then runs alone at a fraction of
    // the SIMD's issue rate.  Each wave lowers its priority by one level per
    // quarter of its share done, so the waves of a SIMD finish together.
    // a wave's share: its chunks of unquantized tokens (last split only),
    // then its groups
    const int chunk0 = split == splits - 1 ? nwaves - 1 - wave : nchunks;
    const int my_chunks = chunk0 < nchunks ? (nchunks - 1 - chunk0) / nwaves + 1 : 0;
    const int my_steps = my_chunks + (gb < g1 ? (g1 - 1 - gb) / stride + 1 : 0);
    // step d is in quarter floor(4 d / my_steps): d >= ceil(k my_steps / 4)
    const int q1 = (my_steps + 3) / 4, q2 = (2 * my_steps + 3) / 4, q3 = (3 * my_steps + 3) / 4;
    int done = 0;
    auto set_priority = [&]() __attribute__((always_inline)) {
        if constexpr (kDynamicGroups)
            return;
        const int quarter = (done >= q1) + (done >= q2) + (done >= q3);
        ++done;
        if (quarter == 0)
            __builtin_amdgcn_s_setprio(3);
        else if (quarter == 1)
            __builtin_amdgcn_s_setprio(2);
        else if (quarter == 2)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
    };
    using Step = StepData<KB, S::NVW, S::NVM>;
    // With kDefer, values lag the keys by one step: a step scores its
    // group's keys and adds the previous group's values, so the first step
    // waits for key words only (half the first burst of loads).
    constexpr bool kDefer = defers_values(KB, VB, QPK, NP);
    float pw_prev[QPK];
    bool has_prev = false;
    // One wave step on the words in `use` while the next step's words load
    // into `fill`; the loop below alternates the two buffers.
    auto step = [&](Step& use, Step& fill) __attribute__((always_inline)) {
        asm volatile("" : "+v"(tw_base));
        set_priority();
        // unconditional (clamped) prefetch of the next step's words:
        // straight-line code lets the compiler wait only for the loads each
        // part uses.  With deferred values, `fill` takes the next step's keys
        // and this step's values, and the previous step's values are added
        // now, with the weights that step computed (relative to the running
        // maximum before this step's rescale).
        int gnew = gb + stride;
        if constexpr (kDynamicGroups) {
            int g = 0;
            if (lane == 0)
                g = atomicAdd(&group_next, S::GPW);
            gnew = __builtin_amdgcn_readfirstlane(g);
        }
        const int gnext = min(gnew, g1 - 1);
        load_keys<D, KB, VB, QPK>(hp, p.rope_group, lane, gnext, g1, fill);
        if constexpr (kDefer) {
            load_values<D, KB, VB, QPK, (S::GPW > 1)>(hp, lane, gb * G, g1 * G - 1, fill.vw,
                                                      fill.vm);
            if (has_prev)
                accumulate_values<D, KB, VB, QPK>(lane, pw_prev, use.vw, use.vm, st);
        } else {
            load_values<D, KB, VB, QPK, (S::GPW > 1)>(hp, lane, gnext * G, g1 * G - 1, fill.vw,
                                                      fill.vm);
        }
        const float s0 = h2f(use.km.x), z0 = h2f(use.km.x >> 16);
        const float s1 = h2f(use.km.y), z1 = h2f(use.km.y >> 16);
        float s[QPK];
        if constexpr (S::ROWDPP) {
            const float2 Q = cmul(qc[0], use.rg);
            // X + iY = Q (x + iy): X = P + a c0 + bb c1, Y = R + dq c0 + e c1
            const float P = Q.x * z0 - Q.y * z1, a = Q.x * s0, bb = -Q.y * s1;
            const float R = Q.y * z0 + Q.x * z1, dq = Q.y * s0, e = Q.x * s1;
            float Ps[KC::NSCALE], Rs[KC::NSCALE];
#pragma unroll
            for (int k = 0; k < KC::NSCALE; ++k) {
                const float sc = 1.0f / (float)(1 << (24 - k * KB));
                Ps[k] = P * sc;
                Rs[k] = R * sc;
            }
            // rotate each 16-token unit right by q tokens (KB * q bits):
            // position d of unit u then holds token 16 u + (d + q) mod 16
            constexpr int WPU = S::WPU;
            const uint32_t q16 = (uint32_t)(lane & 15);
            uint32_t wr[2][2][WPU];  // [channel x, y][unit][word]
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint32_t* w = use.kw + c * S::WK + u * WPU;
                    if constexpr (WPU == 1) {
                        wr[c][u][0] = __builtin_amdgcn_alignbit(w[0], w[0], 2u * q16);
                    } else {
                        const uint64_t x = ((uint64_t)w[1] << 32) | w[0];
                        const uint32_t sh = (uint32_t)KB * q16;  // < 64
                        const uint64_t r = (x >> sh) | (x << ((64u - sh) & 63u));
                        wr[c][u][0] = (uint32_t)r;
                        wr[c][u][1] = (uint32_t)(r >> 32);
                    }
                }
            s[0] = row_dpp_scores([&](int f) __attribute__((always_inline)) {
                const int sidx = KC::pos(f) / KB;
                // field f of each word, both halves from one AND (kept
                // whole, not narrowed per half)
                uint32_t m[2][2][WPU];
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int k = 0; k < WPU; ++k) {
                            const uint32_t w = wr[c][u][k];
                            m[c][u][k] = KC::field(w, w >> KC::SHIFT, f);
                            asm("" : "+v"(m[c][u][k]));
                        }
                auto xy = [&](float c0, float c1) {
                    return make_float2(fmaf(bb, c1, fmaf(a, c0, Ps[sidx])),
                                       fmaf(e, c1, fmaf(dq, c0, Rs[sidx])));
                };
                Terms<NPOS> v;
#pragma unroll
                for (int k = 0; k < WPU; ++k)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        auto half = [&](uint32_t x) { return h ? hi_h(x) : lo_h(x); };
                        const float2 t0 = xy(half(m[0][0][k]), half(m[1][0][k]));
                        const float2 t1 = xy(half(m[0][1][k]), half(m[1][1][k]));
                        v.v[2 * k + h] = make_float4(t0.x, t0.y, t1.x, t1.y);
                    }
                return v;
            });
        } else if constexpr (QPK == 1) {
#pragma unroll
            for (int h = 0; h < QPK; ++h) {
                const float2 Q = cmul(qc[h], use.rg);
                // X = P + a c0 + bb c1 = Re[Q (x+iy)],  Y = R + d c0 + e c1 = Im[Q (x+iy)]
                const float P = Q.x * z0 - Q.y * z1, a = Q.x * s0, bb = -Q.y * s1;
                const float R = Q.y * z0 + Q.x * z1, d = Q.y * s0, e = Q.x * s1;
                float Ps[KC::NSCALE], Rs[KC::NSCALE];
#pragma unroll
                for (int k = 0; k < KC::NSCALE; ++k) {
                    const float sc = 1.0f / (float)(1 << (24 - k * KB));
                    Ps[k] = P * sc;
                    Rs[k] = R * sc;
                }
#pragma unroll
                for (int w = 0; w < S::WK; ++w) {
                    const uint32_t w0 = use.kw[w], w1 = use.kw[S::WK + w];
                    const uint32_t w0s = w0 >> KC::SHIFT, w1s = w1 >> KC::SHIFT;
#pragma unroll
                    for (int f = 0; f < KC::TPH; ++f) {
                        const uint32_t m0 = KC::field(w0, w0s, f), m1 = KC::field(w1, w1s, f);
                        const int sidx = KC::pos(f) / KB;
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int j = w * 2 * KC::TPH + half * KC::TPH + f;
                            const float c0 = half ? hi_h(m0) : lo_h(m0);
                            const float c1 = half ? hi_h(m1) : lo_h(m1);
                            const float X = fmaf(bb, c1, fmaf(a, c0, Ps[sidx]));
                            const float Y = fmaf(e, c1, fmaf(d, c0, Rs[sidx]));
                            const float2 tw = twiddle(j);
                            red[lane * RS + j] = fmaf(tw.x, X, tw.y * Y);
                        }
                    }
                }
                float a4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
                for (int m = 0; m < 32; ++m)
                    a4[m & 3] += red[(red_half + m) * RS + red_col];
                float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
                if (NP == 64)
                    acc = half_sum(acc);
                s[h] = acc;
            }
        } else {
            // Several query heads share the key tile: dequantize and rotate
            // each (pair, token) once, U_j = T_j (x + i y) (times the field
            // scale 2^(pos-24) and its inverse folded into T_j), then each
            // head's term is Re[Q_h U_j] with Q_h = conj(q'_h) e^{i g G theta_i}.
            // With the matrix-core scores, U is formed at 1/4 scale (folded
            // into the dequantization) so that it fits binary16 for any
            // binary16 keys; the queries carry the factor 4.
            constexpr float kUScale = kMfmaHeads ? 0.25f : 1.0f;
            const float s0u = s0 * kUScale, s1u = s1 * kUScale;
            float z0s[KC::NSCALE], z1s[KC::NSCALE];
#pragma unroll
            for (int k = 0; k < KC::NSCALE; ++k) {
                const float sc = kUScale / (float)(1 << (24 - k * KB));
                z0s[k] = z0 * sc;
                z1s[k] = z1 * sc;
            }
            float ux[G], uy[G];
#pragma unroll
            for (int w = 0; w < S::WK; ++w) {
                const uint32_t w0 = use.kw[w], w1 = use.kw[S::WK + w];
                const uint32_t w0s = w0 >> KC::SHIFT, w1s = w1 >> KC::SHIFT;
#pragma unroll
                for (int f = 0; f < KC::TPH; ++f) {
                    const uint32_t m0 = KC::field(w0, w0s, f), m1 = KC::field(w1, w1s, f);
                    const int sidx = KC::pos(f) / KB;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int jj = w * 2 * KC::TPH + half * KC::TPH + f;
                        const float c0 = half ? hi_h(m0) : lo_h(m0);
                        const float c1 = half ? hi_h(m1) : lo_h(m1);
                        const float x = fmaf(s0u, c0, z0s[sidx]);
                        const float y = fmaf(s1u, c1, z1s[sidx]);
                        const float2 tw = twiddle(jj);  // (T.x, -T.y) * 2^(24-pos)
                        ux[jj] = fmaf(tw.x, x, tw.y * y);
                        uy[jj] = fmaf(tw.x, y, -(tw.y * x));
                    }
                }
            }
            if constexpr (kMfmaHeads) {
                // The heads' scores of the step's 32 tokens as one matrix
                // product on the matrix cores: S[h][j] = sum_k A[h][k] B[k][j]
                // over k = 2 i + {0, 1} for the 64 pairs, A[h][2i] = 4 Q_h.x,
                // A[h][2i+1] = -4 Q_h.y, B[2i][j] = U_j.x / 4, B[2i+1][j] =
                // U_j.y / 4 (both inside binary16 for any binary16 inputs).
                // Every operand is split hi + lo (split_h2) and hi*hi + hi*lo
                // + lo*hi accumulate in fp32 in v_mfma_f32_16x16x32_f16.  The
                // operands reach the MFMA lane layouts through this wave's
                // region of the reduce buffers: lane i (pair i) writes one
                // (hi, lo) word pair per head and per token, and each lane
                // reads 16-byte runs of four pairs (16-byte chunks swizzled
                // by row, so the column reads hit distinct banks).  All
                // of it stays inside the wave, whose LDS accesses execute in
                // program order; the compiler barriers keep that order.
                uint32_t* const wsb = reinterpret_cast<uint32_t*>(red);
                uint32_t* const uhi = wsb;             // [16 tokens][kUS]
                uint32_t* const ulo = wsb + 16 * kUS;
                uint32_t* const qhi = wsb + 32 * kUS;  // [QPK heads][kUS]
                uint32_t* const qlo = qhi + QPK * kUS;
                // word c of a row at 16-byte chunk (c / 4) XOR (row % 16):
                // the 16-byte reads of a column of rows fall in distinct banks
                auto swz = [](int row, int c) { return (((c >> 2) ^ (row & 15)) << 2) | (c & 3); };
                float m1 = -1.0f;
                asm volatile("" : "+v"(m1));
#pragma unroll
                for (int h = 0; h < QPK; ++h) {
                    const float2 Q = cmul(qc[h], use.rg);
                    const uint2 w = split_h2(4.0f * Q.x, -4.0f * Q.y, m1);
                    qhi[h * kUS + swz(h, i)] = w.x;
                    qlo[h * kUS + swz(h, i)] = w.y;
                }
                auto store_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const uint2 w = split_h2(ux[16 * t + jj], uy[16 * t + jj], m1);
                        uhi[jj * kUS + swz(jj, i)] = w.x;
                        ulo[jj * kUS + swz(jj, i)] = w.y;
                    }
                };
                store_tile(0);
                asm volatile("" ::: "memory");
                // A: lane (row m = lane % 16, k-run kq = lane / 16); rows
                // past the heads are zero.  B: lane (token column m, kq).
                const int mrow = lane & 15, kq = lane >> 4;
                half8v ahi[4], alo[4];
#pragma unroll
                for (int sk = 0; sk < 4; ++sk) {
                    ahi[sk] = half8v{};
                    alo[sk] = half8v{};
                    if (mrow < QPK) {
                        ahi[sk] = *reinterpret_cast<const half8v*>(qhi + mrow * kUS + swz(mrow, 16 * sk + 4 * kq));
                        alo[sk] = *reinterpret_cast<const half8v*>(qlo + mrow * kUS + swz(mrow, 16 * sk + 4 * kq));
                    }
                }
                float4v acc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (t == 1) {
                        asm volatile("" ::: "memory");
                        store_tile(1);
                        asm volatile("" ::: "memory");
                    }
                    float4v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int sk = 0; sk < 4; ++sk) {
                        const half8v bhi =
                            *reinterpret_cast<const half8v*>(uhi + mrow * kUS + swz(mrow, 16 * sk + 4 * kq));
                        const half8v blo =
                            *reinterpret_cast<const half8v*>(ulo + mrow * kUS + swz(mrow, 16 * sk + 4 * kq));
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sk], bhi, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sk], blo, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[sk], bhi, c, 0, 0, 0);
                    }
                    acc[t] = c;
                }
                asm volatile("" ::: "memory");
                // Lanes 0..15 hold the heads of token `lane` in acc[0] and of
                // token 16 + lane in acc[1]; the softmax wants token lane % 32
                // in lane: row 1 takes row 0's acc[1], rows 2 and 3 rows 0, 1.
                // (Both swaps run in every lane: inside a branch, the lanes
                // they read from would be inactive.)
                const bool row1 = (lane & 16) != 0;
#pragma unroll
                for (int h = 0; h < QPK; ++h) {
                    const float from_row0 = swap16(acc[1][h]).a;
                    const float x = row1 ? from_row0 : acc[0][h];
                    s[h] = swap32(x).a;
                }
            } else {
#pragma unroll
                for (int h = 0; h < QPK; ++h) {
                    // heads alternate between two buffers, so one head's writes
                    // need not wait for the previous head's reads
                    float* rb = red + (S::NRED > 1 ? (h & 1) : 0) * 64 * RS;
                    const float2 Q = cmul(qc[h], use.rg);
                    const float nqy = -Q.y;
#pragma unroll
                    for (int jj = 0; jj < G; ++jj)
                        rb[lane * RS + jj] = fmaf(Q.x, ux[jj], nqy * uy[jj]);
                    float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 32; ++m)
                        a4[m & 3] += rb[(red_half + m) * RS + red_col];
                    float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
                    if (NP == 64)
                        acc = half_sum(acc);
                    s[h] = acc;
                }
            }
        }
        if constexpr (kDefer) {
            softmax_weights<D, KB, VB, QPK>(lane, gb * G, g1 * G, s, pw_prev, st);
            has_prev = true;
        } else {
            softmax_values<D, KB, VB, QPK>(lane, gb * G, g1 * G, s, use.vw, use.vm, st);
        }
        gb = gnew;
    };
    // Unquantized chunks (last split only).  Where the variant's registers
    // allow (chunks_first), they go before the wave's groups and then run
    // beside the other waves' groups, paced by the priorities, instead of
    // alone after them; a wave's first group is loaded after them either
    // way, so no group's words are held in registers across the chunk code.
    auto score_chunks = [&]() __attribute__((always_inline)) {
        for (int ch = chunk0; ch < nchunks; ch += nwaves) {
            asm volatile("" : "+v"(tw_base));  // keep the twiddle reads in the loop
            set_priority();
            // One chunk of unquantized tokens t0 .. t0+cnt-1, from the sinks or
            // the rings (rows from row0, contiguous: the ring and t0 are
            // multiples of G), scored like one more group (the softmax is
            // order-free): lane = channel pair, the tokens across its registers.
            const bool in_sink = ch < nsink_chunks;
            const int t0 = in_sink ? ch * G : tq + (ch - nsink_chunks) * G;
            const int cnt = min(G, (in_sink ? ns : n) - t0);
            const size_t row0 = in_sink ? bh * (size_t)p.sink + t0 : bh * (size_t)p.ring + t0 % p.ring;
            const void* const krows = in_sink ? p.k_sink : p.k_tail;
            // row-DPP sums: register j holds token tok(j), the rotated order
            // of the group step (lane_q opaque: its 32 row offsets are made
            // here, not hoisted out of the chunk loop into held registers)
            int lane_q = lane & 15;
            asm volatile("" : "+v"(lane_q));
            auto tok = [&](int j) { return (j & 16) | ((j + lane_q) & 15); };
            const float2 rg = p.rope_group[(size_t)(t0 / G) * NP + i];
            float s[QPK];
            if constexpr (S::ROWDPP) {
                // registers in the rotated order of the group step; binary16
                // words kept whole and converted where they are used
                const float2 Q = cmul(qc[0], rg);
                auto v4 = [&](float x0, float y0, float x1, float y1, int d) {
                    // Q (x + iy) at the field scale 2^(pos-24) of the
                    // register's word position, which the twiddles undo
                    const float un = 1.0f / (float)(1 << (24 - KC::pos(d % KC::TPH)));
                    return make_float4((Q.x * x0 - Q.y * y0) * un, (Q.x * y0 + Q.y * x0) * un,
                                       (Q.x * x1 - Q.y * y1) * un, (Q.x * y1 + Q.y * x1) * un);
                };
                if (p.dtype == 0) {
                    const uint32_t* t32 = reinterpret_cast<const uint32_t*>(krows) + row0 * (D / 2);
                    uint32_t kr[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const int t = tok(j);
                        kr[j] = t < cnt ? t32[(unsigned)(t * (D / 2) + i)] : 0u;
                    }
                    auto at = [&](int d) {
                        return v4(lo_h(kr[d]), hi_h(kr[d]), lo_h(kr[16 + d]), hi_h(kr[16 + d]), d);
                    };
                    s[0] = row_dpp_scores([&](int f) __attribute__((always_inline)) {
                        Terms<NPOS> v;
#pragma unroll
                        for (int pi = 0; pi < NPOS; ++pi)
                            v.v[pi] = at(pi * KC::TPH + f);
                        return v;
                    });
                } else {
                    const float2* t64 = reinterpret_cast<const float2*>(krows) + row0 * (D / 2);
                    float2 kr[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const int t = tok(j);
                        kr[j] = t < cnt ? t64[(unsigned)(t * (D / 2) + i)] : make_float2(0.f, 0.f);
                    }
                    auto at = [&](int d) {
                        return v4(kr[d].x, kr[d].y, kr[16 + d].x, kr[16 + d].y, d);
                    };
                    s[0] = row_dpp_scores([&](int f) __attribute__((always_inline)) {
                        Terms<NPOS> v;
#pragma unroll
                        for (int pi = 0; pi < NPOS; ++pi)
                            v.v[pi] = at(pi * KC::TPH + f);
                        return v;
                    });
                }
            }
            float tx[G], ty[G];
            if (S::ROWDPP) {
            } else if (p.dtype == 0) {
                // rows of D binary16: a uniform base and a 32-bit lane offset
                const uint32_t* t32 = reinterpret_cast<const uint32_t*>(krows) + row0 * (D / 2);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const uint32_t w =
                        (gsub == 0 && j < cnt) ? t32[(unsigned)(j * (D / 2) + i)] : 0u;
                    tx[j] = lo_h(w);
                    ty[j] = hi_h(w);
                }
            } else {
                const float2* t64 = reinterpret_cast<const float2*>(krows) + row0 * (D / 2);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const float2 w = (gsub == 0 && j < cnt) ? t64[(unsigned)(j * (D / 2) + i)]
                                                            : make_float2(0.f, 0.f);
                    tx[j] = w.x;
                    ty[j] = w.y;
                }
            }
#pragma unroll
            for (int h = 0; h < (S::ROWDPP ? 0 : QPK); ++h) {
                const float2 Q = cmul(qc[h], rg);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    // Re[T_j Q (x + iy)]; the twiddle carries (T.x, -T.y) * 2^(24-pos)
                    const float vr = Q.x * tx[j] - Q.y * ty[j];
                    const float vi = Q.x * ty[j] + Q.y * tx[j];
                    const float unscale = 1.0f / (float)(1 << (24 - KC::pos(j % KC::TPH)));
                    const float2 tw = twiddle(j);
                    red[lane * RS + j] = fmaf(tw.x, vr, tw.y * vi) * unscale;
                }
                float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 32; ++m)
                    a4[m & 3] += red[(red_half + m) * RS + red_col];
                float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
                if (NP == 64)
                    acc = half_sum(acc);
                s[h] = acc;
            }
            if (in_sink || p.residual > 0) {
                const char* vrows = static_cast<const char*>(in_sink ? p.v_sink : p.v_tail) +
                                    row0 * D * (p.dtype == 0 ? 2 : 4);
                softmax_fp_values<D, KB, VB, QPK>(lane, t0, cnt, s, vrows, p.dtype, st);
            } else {
                uint32_t vw[S::NVW], vm[S::NVM];
                load_values<D, KB, VB, QPK, true>(hp, lane, t0, n - 1, vw, vm);
                softmax_values<D, KB, VB, QPK>(lane, t0, n, s, vw, vm, st);
            }
        }
    };
    if constexpr (chunks_first(KB, VB, QPK))
        score_chunks();
    if (gb < g1) {
        load_keys<D, KB, VB, QPK>(hp, p.rope_group, lane, gb, g1, cur);
        if constexpr (!kDefer)
            load_values<D, KB, VB, QPK, (S::GPW > 1)>(hp, lane, gb * G, g1 * G - 1, cur.vw,
                                                      cur.vm);
    }
    bool last_in_nxt = false;  // which buffer holds the last step's values
    while (gb < g1) {
        step(cur, nxt);
        last_in_nxt = true;
        if (gb >= g1)
            break;
        step(nxt, cur);
        last_in_nxt = false;
    }
    if (kDefer && has_prev)
        accumulate_values<D, KB, VB, QPK>(lane, pw_prev, last_in_nxt ? nxt.vw : cur.vw,
                                          last_in_nxt ? nxt.vm : cur.vm, st);
    if constexpr (!chunks_first(KB, VB, QPK))  // the same chunks, after the groups
        score_chunks();

    __builtin_amdgcn_s_setprio(0);

    // ---- merge the waves of this block.  The merge area overlaps the
    // reduce buffers, so every wave must be done with its own first; the
    // row-DPP variants have none (nothing but the twiddles is in LDS during
    // their loop), so a wave that finishes early reduces and stores its
    // state at once, while the others still run.
    if constexpr (!S::ROWDPP)
        __syncthreads();
    float* sm = smem;                           // [nwaves][QPK]
    float* sl = smem + kMaxWaves * QPK;         // [nwaves][QPK]
    float* so = smem + 2 * kMaxWaves * QPK;     // [nwaves][QPK][D]
    if constexpr (S::PAIRS) {
        // lane (r, c) holds channel group r over its tokens: sum the 16
        // lanes of row r per channel by halving exchanges -- at each stage
        // a lane keeps half of its channels and adds its partner's values
        // of that half (partners: mirror, half mirror, xor 2, xor 1, each
        // pairing lanes that differ in bit 3, 2, 1, 0), so lane c ends with
        // channels 2c and 2c + 1 of the group.  The zero-point terms are the
        // same for every channel of the row: summed once.
        const float L = wave_sum(st.l[0]);
        const int r = lane >> 4, c16 = lane & 15;
        float zs = st.z[0];
        zs += dpp<kDppXor1>(zs);
        zs += dpp<kDppXor2>(zs);
        zs += dpp<kDppHalfMirror>(zs);
        zs += dpp<kDppMirror>(zs);
        float v[G];
#pragma unroll
        for (int c = 0; c < G; ++c)
            v[c] = st.o[0][c];
        auto halve = [&](auto ctrl, int half, bool upper) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < half; ++i) {
                const float keep = upper ? v[i + half] : v[i];
                const float send = upper ? v[i] : v[i + half];
                v[i] = keep + dpp_all<decltype(ctrl)::value>(send);
            }
        };
        halve(std::integral_constant<int, kDppMirror>{}, 16, (c16 & 8) != 0);
        halve(std::integral_constant<int, kDppHalfMirror>{}, 8, (c16 & 4) != 0);
        halve(std::integral_constant<int, kDppXor2>{}, 4, (c16 & 2) != 0);
        halve(std::integral_constant<int, kDppXor1>{}, 2, (c16 & 1) != 0);
        float2 x;
        x.x = fmaf(v[0], (float)(1 << (24 - VC::pos((2 * c16) % VC::TPH))), zs);
        x.y = fmaf(v[1], (float)(1 << (24 - VC::pos((2 * c16 + 1) % VC::TPH))), zs);
        *reinterpret_cast<float2*>(so + wave * D + r * G + 2 * c16) = x;
        if (lane == 0) {
            sm[wave] = st.m[0];
            sl[wave] = L;
        }
    } else if constexpr (S::QUADS) {
        // lane (r, c) holds words (2r + c/8) * NW.. over its tokens: sum the
        // 8 lanes that share them (c & 7 = 0..7)
        const int w0 = (2 * (lane >> 4) + ((lane & 15) >> 3)) * S::NW;
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const float L = wave_sum(st.l[h]);
#pragma unroll
            for (int c = 0; c < S::NCL; ++c) {
                const float sc = (float)(1 << (24 - VC::pos(c % VC::TPH)));
                float x = fmaf(st.o[h][c], sc, st.z[h]);
                x += dpp<kDppXor1>(x);
                x += dpp<kDppXor2>(x);
                x += dpp<kDppHalfMirror>(x);
                if ((lane & 7) == 0)
                    so[(wave * QPK + h) * D + w0 * S::NC + c] = x;
            }
            if (lane == 0) {
                sm[wave * QPK + h] = st.m[h];
                sl[wave * QPK + h] = L;
            }
        }
    } else {
        const int vw = lane % S::WPT, vslot = lane / S::WPT;
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
            const float L = wave_sum(st.l[h]);
            float v[S::NC];
#pragma unroll
            for (int c = 0; c < S::NC; ++c) {
                // undo the field scale 2^(pos-24) of channel c of the word
                const float sc = (float)(1 << (24 - VC::pos(c % VC::TPH)));
                float x = fmaf(st.o[h][c], sc, st.z[h]);
#pragma unroll
                for (int off = S::WPT; off < 64; off <<= 1)
                    x += __shfl_xor(x, off);
                v[c] = x;
            }
            if (vslot == 0) {
#pragma unroll
                for (int c = 0; c < S::NC; ++c)
                    so[(wave * QPK + h) * D + vw * S::NC + c] = v[c];
            }
            if (lane == 0) {
                sm[wave * QPK + h] = st.m[h];
                sl[wave * QPK + h] = L;
            }
        }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    const bool single = (splits == 1);
    for (int idx = tid; idx < QPK * D; idx += blockDim.x) {
        const int h = idx / D, c = idx % D;
        float M = -INFINITY;
        float L = 0.f, acc = 0.f;
        if constexpr (S::ROWDPP) {
            // unrolled to the largest block, waves past nwaves reading wave
            // 0's slots and weighing nothing, so all the reads issue at once
            constexpr int kW = max_block_waves(QPK);
            float mw[kW], lw[kW], ow[kW];
#pragma unroll
            for (int w = 0; w < kW; ++w) {
                const int ww = w < nwaves ? w : 0;
                mw[w] = w < nwaves ? sm[ww * QPK + h] : -INFINITY;
                lw[w] = sl[ww * QPK + h];
                ow[w] = so[(ww * QPK + h) * D + c];
                M = fmaxf(M, mw[w]);
            }
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kW; ++w) {
                    const float f = exp2f(mw[w] - M);
                    L += f * lw[w];
                    acc += f * ow[w];
                }
            }
        } else {
            for (int w = 0; w < nwaves; ++w)
                M = fmaxf(M, sm[w * QPK + h]);
            if (M != -INFINITY) {
                for (int w = 0; w < nwaves; ++w) {
                    const float f = exp2f(sm[w * QPK + h] - M);
                    L += f * sl[w * QPK + h];
                    acc += f * so[(w * QPK + h) * D + c];
                }
            }
        }
        const size_t row = (size_t)b * p.hq + head0 + h;
        if (single) {
            out[row * D + c] = acc / L;
        } else {
            float* dst = p.partials + (row * p.max_splits + split) * (D + 2);
            dst[c] = acc;
            if (c == 0) {
                dst[D] = M;
                dst[D + 1] = L;
            }
        }
    }
}

// Merge the split partials of one output row (grid: batch * q_heads rows,
// head_dim threads): out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Splits go in chunks of kChunk whose loads all issue before any is used
// (a slot past the last split reads the chunk's first split again with
// m = -inf), merged online.  A split whose m is -inf (no tokens; its o and
// l are stored as 0) or a slot past the end gets the weight 2^-inf = 0
// exactly, so with at most kChunk splits the sums equal those of the
// two-pass form that skips such splits.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const float* __restrict__ partials,
                                                    int max_splits, int splits,
                                                    float* __restrict__ out)
{
    constexpr int kChunk = 8;
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const float* base = partials + row * max_splits * (D + 2);
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kChunk) {
        float mv[kChunk], lv[kChunk], ov[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const bool in = s0 + u < splits;
            const float* b = base + (size_t)(in ? s0 + u : s0) * (D + 2);
            mv[u] = in ? b[D] : -INFINITY;
            lv[u] = b[D + 1];
            ov[u] = b[c];
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < kChunk; ++u)
            Mn = fmaxf(Mn, mv[u]);
        // reference maximum: 0 while no split so far saw tokens (all weights
        // 0 then); the earlier chunks' sums rescale by 2^(M - Mn), which is
        // 0 when M = -inf (the sums are still 0) and 1 when Mn = M
        const float Mr = Mn == -INFINITY ? 0.f : Mn;
        const float r = exp2f(M - Mr);
        L *= r;
        acc *= r;
        M = Mn;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float f = exp2f(mv[u] - Mr);
            L += f * lv[u];
            acc += f * ov[u];
        }
    }
    out[row * D + c] = acc / L;
}

// Bytes of dynamic LDS for a block of nwaves waves.
template <int D, int KB, int VB, int QPK>
constexpr size_t attend_lds_bytes(int nwaves)
{
    using S = Shape<D, KB, VB, QPK>;
    const size_t red = (size_t)nwaves * S::NRED * 64 * S::RED_STRIDE;
    const size_t merge = 2 * kMaxWaves * QPK + (size_t)nwaves * QPK * D;
    return 4 * (red > merge ? red : merge);
}

template <int D, int KB, int VB, int QPK>
void launch(const Planes& p, const void* q, float* out, int n, int splits, int nwaves,
            const void* k_new, const void* v_new, hipStream_t stream)
{
    const int hgroups = p.hq / p.hkv / QPK;
    dim3 grid(splits, p.nb * p.hkv * hgroups);
    nwaves = nwaves < max_block_waves(QPK) ? nwaves : max_block_waves(QPK);
    attend_kernel<D, KB, VB, QPK><<<grid, 64 * nwaves, attend_lds_bytes<D, KB, VB, QPK>(nwaves),
                                    stream>>>(p, q, out, n, splits, hgroups, k_new, v_new);
    if (splits > 1)
        combine_kernel<D><<<p.nb * p.hq, D, 0, stream>>>(p.partials, p.max_splits, splits, out);
}

template <int D, int KB, int VB>
void by_qpk(const Planes& p, const void* q, float* out, int n, int splits, int nwaves,
            const void* k_new, const void* v_new, hipStream_t s)
{
    switch (p.hq / p.hkv) {
    case 1: launch<D, KB, VB, 1>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 2: launch<D, KB, VB, 2>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 4:  // 8 query heads per KV head run as two groups of 4 (registers)
    case 8: launch<D, KB, VB, 4>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    }
}

template <int D, int KB>
void by_vb(const Planes& p, const void* q, float* out, int n, int splits, int nwaves,
           const void* k_new, const void* v_new, hipStream_t s)
{
    switch (p.vbits) {
    case 2: by_qpk<D, KB, 2>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 4: by_qpk<D, KB, 4>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 8: by_qpk<D, KB, 8>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    }
}

template <int D>
hipError_t launch_attend_d(const Planes& p, const void* q, float* out, int n, int splits,
                           int nwaves, const void* k_new, const void* v_new, hipStream_t s)
{
    switch (p.kbits) {
    case 2: by_vb<D, 2>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 4: by_vb<D, 4>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    case 8: by_vb<D, 8>(p, q, out, n, splits, nwaves, k_new, v_new, s); break;
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace kvqi
