/*
 * oracle.c -- plain, slow, single-threaded fp64 reference for KIVI-style
 * asymmetric KV-cache quantization and the decode attention that reads the
 * quantized cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the package's smoke check and the bench's
 * CPU-baseline leg do.  It includes no HIP header and shares no source with
 * the GPU library.
 *
 * Sources (web pages), cited as:
 *   [GEOM]  "Why KV Cache Geometry Matters More Than Bit Precision for LLM
 *           Speed" (milik.ai)
 *   [BITS]  "Your KV Cache Doesn't Have a Bit Problem. It Has a Geometry
 *           Problem" (Unite.AI article, tastytech.in repost)
 *   [ROT]   "Rotate, Then Round: The Geometry of KV-Cache Compression"
 *           (aissential.tech digest)
 *
 * What is computed, step by step (every floating-point step in fp64):
 *   1. Quantize one group of values (uniform asymmetric integer code):
 *      zero point = group minimum, step = range / (2^B - 1), each element
 *      rounded to the nearest step.  [BITS, "What Quantization Error Is
 *      Actually Made Of"]; [GEOM, "Inside the Attention Equation"].
 *      Readings where the pages are silent: ties go to the even code; the
 *      zero and the step are stored as IEEE binary16, each rounded once
 *      (round-to-nearest-even) from the exact value; codes are computed
 *      against the stored binary16 zero and step; a zero step gives code 0.
 *   2. Keys are grouped per channel over runs of G consecutive tokens,
 *      values per token over runs of G consecutive channels.  [BITS, "Keys:
 *      The Outliers Live in Fixed Channels", "Values: Where the Intuition
 *      Breaks"]; [GEOM, "Stop Obsessing Over Bits"].
 *   3. Key tokens that do not yet fill a G-token group stay unquantized in
 *      a tail buffer.  [BITS, "The Systems Tax, and Why It Is Not a Detail"].
 *      Residual window R (KIVI keeps the most recent tokens in full
 *      precision; [BITS], same section): with R > 0, keys and values of
 *      tokens [Tq, n) stay unquantized, Tq = G * floor(max(0, n - R) / G), so
 *      at least R (at most R + G - 1) recent tokens; a G-block is quantized
 *      when it leaves the window.  R = 0: Tq = G * floor(n / G) for keys and
 *      every value is quantized on arrival.
 *      Sink window S (InnerQ keeps high-precision windows for recent and
 *      attention-sink tokens; [BITS, "Where the Work Is Headed"]): keys and values of tokens [0, min(n, S)) stay
 *      unquantized for good; the quantized region starts at S (a multiple of
 *      G, so key groups stay aligned to token 0) and Tq is raised to at
 *      least min(n, S).
 *   4. Keys are stored before the rotary position embedding; the rotation is
 *      applied after dequantization.  [BITS, "Rotary Embeddings Complicate
 *      the Keys"]; [GEOM, "What Data Scientists Should Do Next"].
 *      Reading: channels (2i, 2i+1) form a pair (neighbouring channels), the
 *      pair rotates by p * theta_i with theta_i = base^(-2i/D); the query is
 *      rotated at position n-1.
 *   5. Attention output = softmax-weighted sum of the value vectors over all
 *      cached tokens, scores scaled by 1/sqrt(D).  [BITS, "Values: Where the
 *      Intuition Breaks"].  Softmax is the plain two-pass form.
 *   7. FP8 cache ([ROT], "Key Takeaways" and the practical guidance: FP8 is
 *      the production default at 2x capacity): every key and value element
 *      stored as one OCP FP8 E4M3 byte (1 sign, 4 exponent bits with bias 7,
 *      3 mantissa bits; largest finite 448; no infinities).  Readings: no
 *      scale factor (scale 1); round to nearest, ties to even, values beyond
 *      the largest finite saturate to +-448; keys stored before the rotary
 *      embedding like the integer cache.  Planes here are in the logical
 *      order [nb][Hkv][Gcap][D][32]: inside each 32-token group the byte of
 *      channel c, token j sits at c * 32 + j.  (The pages fix no byte order;
 *      the GPU library keeps the same bytes in an order of its own, and the
 *      tests permute its planes to this one before comparing.)
 *   6. Geometry ablation ([BITS], lede and "Keys: The Outliers Live in Fixed
 *      Channels", "Values: Where the Intuition Breaks"): the same 2 bits
 *      spent along the other axis -- keys per token (a group is G channels
 *      of one token, quantized on arrival) and/or values per channel (a group
 *      is one channel over G tokens; unfilled value groups wait in a tail
 *      like the keys').  The planes of a flipped operand take the other
 *      operand's layout.  Error where it is consumed, against the unquantized
 *      inputs (reading: per output row, i.e. per (sequence, query head), then
 *      averaged over rows): key and value reconstruction error (Frobenius
 *      norm over the row's KV head), attention-score error (L2 norm of the
 *      difference of the softmax weights from stored and from unquantized
 *      keys), the value side's relative output error (weights from
 *      unquantized keys, stored against unquantized values) and the
 *      end-to-end relative output error.
 *
 * Packed layout (the bit-exact contract shared with the GPU library, which
 * implements it separately):
 *   K_CODES u32[nb][Hkv][Gcap][D][Wk]   Wk = G*Bk/32; token j of a group at
 *                                       bits [j*Bk, j*Bk+Bk) of the group's
 *                                       little-endian bit string for channel c
 *   K_META  u32[nb][Hkv][Gcap][D]       binary16 step | binary16 zero << 16
 *   V_CODES u32[nb][Hkv][Tcap][D/G][Wv] channel j of a channel group at bits
 *                                       [j*Bv, j*Bv+Bv)
 *   V_META  u32[nb][Hkv][Tcap][D/G]     binary16 step | binary16 zero << 16
 *   K_TAIL  dtype[nb][Hkv][R+G][D]      ring: token t >= Tq in slot t mod (R+G),
 *                                       verbatim (R = 0: slot t - Tq)
 *   V_TAIL  dtype[nb][Hkv][R+G][D]      the same for values (R > 0 only)
 *   K_SINK  dtype[nb][Hkv][S][D]        token t < min(n, S) in slot t
 *   V_SINK  dtype[nb][Hkv][S][D]        the same for values
 *
 * Input element types: ORC_F16 (IEEE binary16 bit patterns) or ORC_F32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F16 0
#define ORC_F32 1

/* ---------------------------------------------------------------- binary16 */

/* binary16 -> double, from the IEEE 754 definition of the format. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* double -> binary16 with one rounding, to nearest, ties to even,
 * subnormals included, overflow to infinity.  The value is scaled by a power
 * of two so that one binary16 quantum becomes 1, rounded with nearbyint in the
 * default (to-nearest-even) mode, and re-encoded. */
uint16_t orc_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    /* 65504 is the largest finite value; its quantum is 32, so the halfway
     * point to the next binade is 65520, which rounds to even (infinity). */
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
    int quantum = (e - 1) - 10; /* exponent of one unit in the last place */
    if (quantum < -24)
        quantum = -24;          /* subnormal range: fixed quantum 2^-24 */
    double r = nearbyint(ldexp(a, -quantum));
    double v = ldexp(r, quantum); /* the rounded magnitude */
    if (v == 0.0)
        return sign;
    int e2;
    frexp(v, &e2);
    int E = e2 - 1; /* v in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal: v = m * 2^-24 */
        return sign | (uint16_t)ldexp(v, 24);
    }
    if (E > 15)
        return sign | 0x7c00;
    uint16_t mant = (uint16_t)(ldexp(v, -E) * 1024.0 - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | mant;
}

static double load_elem(const void* p, int dtype, size_t i)
{
    if (dtype == ORC_F16)
        return orc_half_to_double(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* ------------------------------------------------------------ quantizer */

/* Quantize one group of n values with B-bit codes.
 * [BITS, "What Quantization Error Is Actually Made Of"]: record the smallest
 * value as the zero point, divide the group's range by 2^B - 1 to get the
 * step, round every element to the nearest step.
 * Returns 0, or -1 on bad arguments. */
int orc_quant_group(const double* x, int n, int bits, uint8_t* codes,
                    uint16_t* s16_out, uint16_t* z16_out)
{
    if (n <= 0 || bits < 1 || bits > 8)
        return -1;
    double mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    double levels = (double)((1 << bits) - 1);
    uint16_t z16 = orc_double_to_half(mn);
    /* (mx - mn) is exact in fp64 for binary16 and ordinary fp32 inputs; the
     * fp64 quotient never lands on the wrong side of a binary16 rounding
     * boundary for such inputs, so this equals one rounding of the exact
     * quotient. */
    uint16_t s16 = orc_double_to_half((mx - mn) / levels);
    double z = orc_half_to_double(z16);
    double s = orc_half_to_double(s16);
    int top = (1 << bits) - 1;
    for (int i = 0; i < n; ++i) {
        int c = 0;
        if (s != 0.0) {
            double r = nearbyint((x[i] - z) / s); /* nearest, ties to even */
            if (r < 0.0) r = 0.0;
            if (r > (double)top) r = (double)top;
            c = (int)r;
        }
        codes[i] = (uint8_t)c;
    }
    *s16_out = s16;
    *z16_out = z16;
    return 0;
}

/* Pack n codes of `bits` bits, code j at bit offset j*bits of a little-endian
 * bit string made of 32-bit words.  The word array must hold n*bits/32 words
 * (n*bits a multiple of 32). */
void orc_pack(const uint8_t* codes, int n, int bits, uint32_t* words)
{
    int nw = n * bits / 32;
    for (int w = 0; w < nw; ++w)
        words[w] = 0;
    for (int j = 0; j < n; ++j) {
        int bit = j * bits;
        words[bit / 32] |= (uint32_t)codes[j] << (bit % 32);
    }
}

/* Code j of a packed bit string (inverse of orc_pack for one element). */
int orc_code_at(const uint32_t* words, int j, int bits)
{
    int bit = j * bits;
    return (int)((words[bit / 32] >> (bit % 32)) & ((1u << bits) - 1u));
}

void orc_unpack(const uint32_t* words, int n, int bits, uint8_t* codes)
{
    for (int j = 0; j < n; ++j)
        codes[j] = (uint8_t)orc_code_at(words, j, bits);
}

/* First token of the unquantized region of a cache of n tokens with
 * residual window R (step 3 above). */
int orc_quantized_tokens(int n, int G, int R)
{
    int a = n - R;
    return a > 0 ? (a / G) * G : 0;
}

/* The same with a sink window S: tokens [0, min(n, S)) are sink tokens,
 * [S, Tq) quantized, [Tq, n) in the tail ring. */
int orc_quantized_end(int n, int G, int R, int S)
{
    int s = n < S ? n : S;
    int q = orc_quantized_tokens(n, G, R);
    return q > s ? q : s;
}

/* Key planes for T cached tokens with residual window R: groups g < Tq/G
 * are quantized per channel (group = one channel over tokens gG .. gG+G-1);
 * tokens t >= Tq are copied verbatim into ring slot t mod (R+G) of the tail.
 * Planes sized for gcap groups. */
int orc_quantize_keys(const void* k, int dtype, int nb, int hkv, int T, int D,
                      int G, int bits, int R, int S, int gcap, uint32_t* k_codes,
                      uint32_t* k_meta, void* k_tail, void* k_sink)
{
    if (G <= 0 || (G * bits) % 32 != 0 || T < 0 || R < 0 || R % G != 0 ||
        S < 0 || S % G != 0 || (S > 0 && !k_sink) || T / G > gcap)
        return -1;
    int wk = G * bits / 32;
    int tq = orc_quantized_end(T, G, R, S);
    int ngroups = tq / G;
    int ring = R + G;
    int ns = T < S ? T : S;
    size_t esz = (dtype == ORC_F16) ? 2 : 4;
    double* x = (double*)malloc(sizeof(double) * (size_t)G);
    uint8_t* codes = (uint8_t*)malloc((size_t)G);
    if (!x || !codes) {
        free(x);
        free(codes);
        return -2;
    }
    for (int b = 0; b < nb; ++b)
        for (int h = 0; h < hkv; ++h) {
            size_t bh = (size_t)b * hkv + h;
            for (int g = S / G; g < ngroups; ++g)
                for (int c = 0; c < D; ++c) {
                    for (int j = 0; j < G; ++j)
                        x[j] = load_elem(k, dtype,
                                         (bh * T + (size_t)g * G + j) * D + c);
                    uint16_t s16, z16;
                    orc_quant_group(x, G, bits, codes, &s16, &z16);
                    size_t gc = (bh * gcap + g) * D + c;
                    orc_pack(codes, G, bits, k_codes + gc * wk);
                    k_meta[gc] = (uint32_t)s16 | ((uint32_t)z16 << 16);
                }
            for (int t = tq; t < T; ++t)
                memcpy((char*)k_tail + ((bh * ring + t % ring) * D) * esz,
                       (const char*)k + ((bh * T + t) * D) * esz, esz * D);
            for (int t = 0; t < ns; ++t)
                memcpy((char*)k_sink + ((bh * S + t) * D) * esz,
                       (const char*)k + ((bh * T + t) * D) * esz, esz * D);
        }
    free(x);
    free(codes);
    return 0;
}

/* Value planes for T tokens, per channel group (group = channels
 * cg*G .. cg*G+G-1 of one token).  R = 0: every token is quantized.  R > 0:
 * tokens t < Tq are quantized and tokens t >= Tq copied verbatim into ring
 * slot t mod (R+G) of v_tail. */
int orc_quantize_values(const void* v, int dtype, int nb, int hkv, int T,
                        int D, int G, int bits, int R, int S, int tcap,
                        uint32_t* v_codes, uint32_t* v_meta, void* v_tail,
                        void* v_sink)
{
    if (G <= 0 || D % G != 0 || (G * bits) % 32 != 0 || T < 0 || T > tcap ||
        R < 0 || R % G != 0 || (R > 0 && !v_tail) || S < 0 || S % G != 0 ||
        (S > 0 && !v_sink))
        return -1;
    int wv = G * bits / 32;
    int ncg = D / G;
    int tq = R > 0 ? orc_quantized_end(T, G, R, S) : T;
    int ns = T < S ? T : S;
    int ring = R + G;
    size_t esz = (dtype == ORC_F16) ? 2 : 4;
    double* x = (double*)malloc(sizeof(double) * (size_t)G);
    uint8_t* codes = (uint8_t*)malloc((size_t)G);
    if (!x || !codes) {
        free(x);
        free(codes);
        return -2;
    }
    for (int b = 0; b < nb; ++b)
        for (int h = 0; h < hkv; ++h) {
            size_t bh = (size_t)b * hkv + h;
            for (int t = ns; t < tq; ++t)
                for (int cg = 0; cg < ncg; ++cg) {
                    for (int j = 0; j < G; ++j)
                        x[j] = load_elem(v, dtype,
                                         (bh * T + t) * D + (size_t)cg * G + j);
                    uint16_t s16, z16;
                    orc_quant_group(x, G, bits, codes, &s16, &z16);
                    size_t tc = (bh * tcap + t) * ncg + cg;
                    orc_pack(codes, G, bits, v_codes + tc * wv);
                    v_meta[tc] = (uint32_t)s16 | ((uint32_t)z16 << 16);
                }
            for (int t = tq; t < T; ++t)
                memcpy((char*)v_tail + ((bh * ring + t % ring) * D) * esz,
                       (const char*)v + ((bh * T + t) * D) * esz, esz * D);
            for (int t = 0; t < ns; ++t)
                memcpy((char*)v_sink + ((bh * S + t) * D) * esz,
                       (const char*)v + ((bh * T + t) * D) * esz, esz * D);
        }
    free(x);
    free(codes);
    return 0;
}

/* ------------------------------------------------------------------ RoPE */

/* Rotate vector u (length D, D even) in place to position p: the channel
 * pair (2i, 2i+1) turns by the angle p * base^(-2i/D).
 * [BITS, "Rotary Embeddings Complicate the Keys"]. */
void orc_rope(double* u, int D, double p, double base)
{
    for (int i = 0; i < D / 2; ++i) {
        double theta = pow(base, -2.0 * i / (double)D);
        double a = p * theta;
        double c = cos(a), s = sin(a);
        double u0 = u[2 * i], u1 = u[2 * i + 1];
        u[2 * i] = u0 * c - u1 * s;
        u[2 * i + 1] = u0 * s + u1 * c;
    }
}

/* ------------------------------------------------------------- attention */

static double dequant(uint32_t meta, int code)
{
    double s = orc_half_to_double((uint16_t)(meta & 0xffff));
    double z = orc_half_to_double((uint16_t)(meta >> 16));
    return z + s * (double)code;
}

/* Softmax-weighted sum over n tokens given their scores and a callback-free
 * value table (n x D doubles).  Two-pass softmax. */
static void softmax_sum(const double* score, const double* vals, int n, int D,
                        double* out)
{
    double m = score[0];
    for (int t = 1; t < n; ++t)
        if (score[t] > m) m = score[t];
    double l = 0.0;
    for (int c = 0; c < D; ++c)
        out[c] = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(score[t] - m);
        l += w;
        for (int c = 0; c < D; ++c)
            out[c] += w * vals[(size_t)t * D + c];
    }
    for (int c = 0; c < D; ++c)
        out[c] /= l;
}

/* Decode attention over the quantized cache of n tokens (the planes above),
 * for the output rows r in [row_begin, row_end), r = b*Hq + hq.  Query head
 * hq reads KV head hq / (Hq/Hkv).  out holds (row_end-row_begin) x D doubles.
 *   keys and values t < min(n, S): sink slot t (keys rotated to position t);
 *   keys S <= t < Tq: dequantize per channel group, rotate to position t;
 *   keys t >= Tq: tail ring slot t mod (R+G), rotated to position t;
 *   values S <= t < Tq (all t >= S when R = 0): dequantize; else v_tail;
 *   query: rotated to position n-1;
 *   score_t = q'.k'_t / sqrt(D); out = sum_t softmax(score)_t * vhat_t. */
int orc_attend(int nb, int hq, int hkv, int D, int G, int kbits, int vbits,
               int R, int S, int gcap, int tcap, double base,
               const uint32_t* k_codes, const uint32_t* k_meta,
               const void* k_tail, const void* k_sink, const uint32_t* v_codes,
               const uint32_t* v_meta, const void* v_tail, const void* v_sink,
               int dtype, const void* q, int n, int row_begin, int row_end,
               double* out)
{
    if (n <= 0 || hkv <= 0 || hq % hkv != 0 || D % 2 != 0 || D % G != 0 ||
        n > tcap || n / G > gcap || row_begin < 0 || row_end > nb * hq ||
        R < 0 || R % G != 0 || (R > 0 && !v_tail) || S < 0 || S % G != 0 ||
        (S > 0 && (!k_sink || !v_sink)))
        return -1;
    int wk = G * kbits / 32, wv = G * vbits / 32, ncg = D / G;
    int tq = orc_quantized_end(n, G, R, S);
    int vq = R > 0 ? tq : n;
    int ns = n < S ? n : S;
    int ring = R + G;
    double* score = (double*)malloc(sizeof(double) * (size_t)n);
    double* vals = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)D);
    uint8_t* codes = (uint8_t*)malloc((size_t)G);
    if (!score || !vals || !qr || !kr || !codes) {
        free(score); free(vals); free(qr); free(kr); free(codes);
        return -2;
    }
    int group = hq / hkv;
    for (int r = row_begin; r < row_end; ++r) {
        int b = r / hq, h = r % hq, kvh = h / group;
        size_t bh = (size_t)b * hkv + kvh;
        for (int c = 0; c < D; ++c)
            qr[c] = load_elem(q, dtype, (size_t)r * D + c);
        orc_rope(qr, D, (double)(n - 1), base);
        for (int t = 0; t < n; ++t) {
            if (t < ns) {
                for (int c = 0; c < D; ++c)
                    kr[c] = load_elem(k_sink, dtype, (bh * S + t) * D + c);
            } else if (t < tq) {
                int g = t / G, j = t % G;
                for (int c = 0; c < D; ++c) {
                    size_t gc = (bh * gcap + g) * D + c;
                    kr[c] = dequant(k_meta[gc],
                                    orc_code_at(k_codes + gc * wk, j, kbits));
                }
            } else {
                for (int c = 0; c < D; ++c)
                    kr[c] = load_elem(k_tail, dtype,
                                      (bh * ring + t % ring) * D + c);
            }
            orc_rope(kr, D, (double)t, base);
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += qr[c] * kr[c];
            score[t] = dot / sqrt((double)D);
            if (t < ns) {
                for (int c = 0; c < D; ++c)
                    vals[(size_t)t * D + c] =
                        load_elem(v_sink, dtype, (bh * S + t) * D + c);
            } else if (t < vq) {
                for (int cg = 0; cg < ncg; ++cg) {
                    size_t tc = (bh * tcap + t) * ncg + cg;
                    orc_unpack(v_codes + tc * wv, G, vbits, codes);
                    for (int j = 0; j < G; ++j)
                        vals[(size_t)t * D + cg * G + j] =
                            dequant(v_meta[tc], codes[j]);
                }
            } else {
                for (int c = 0; c < D; ++c)
                    vals[(size_t)t * D + c] =
                        load_elem(v_tail, dtype, (bh * ring + t % ring) * D + c);
            }
        }
        softmax_sum(score, vals, n, D, out + (size_t)(r - row_begin) * D);
    }
    free(score); free(vals); free(qr); free(kr); free(codes);
    return 0;
}

/* The same attention over unquantized keys and values k, v laid out
 * [nb][Hkv][n][D] (the full-precision reference a quantized cache should
 * approach as the bit width grows). */
int orc_attend_dense(int nb, int hq, int hkv, int D, double base,
                     const void* k, const void* v, int dtype, const void* q,
                     int n, int row_begin, int row_end, double* out)
{
    if (n <= 0 || hkv <= 0 || hq % hkv != 0 || D % 2 != 0 || row_begin < 0 ||
        row_end > nb * hq)
        return -1;
    double* score = (double*)malloc(sizeof(double) * (size_t)n);
    double* vals = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)D);
    if (!score || !vals || !qr || !kr) {
        free(score); free(vals); free(qr); free(kr);
        return -2;
    }
    int group = hq / hkv;
    for (int r = row_begin; r < row_end; ++r) {
        int b = r / hq, h = r % hq, kvh = h / group;
        size_t bh = (size_t)b * hkv + kvh;
        for (int c = 0; c < D; ++c)
            qr[c] = load_elem(q, dtype, (size_t)r * D + c);
        orc_rope(qr, D, (double)(n - 1), base);
        for (int t = 0; t < n; ++t) {
            for (int c = 0; c < D; ++c) {
                kr[c] = load_elem(k, dtype, (bh * n + t) * D + c);
                vals[(size_t)t * D + c] = load_elem(v, dtype, (bh * n + t) * D + c);
            }
            orc_rope(kr, D, (double)t, base);
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += qr[c] * kr[c];
            score[t] = dot / sqrt((double)D);
        }
        softmax_sum(score, vals, n, D, out + (size_t)(r - row_begin) * D);
    }
    free(score); free(vals); free(qr); free(kr);
    return 0;
}

/* ------------------------------------------------------ geometry ablation */

#define ORC_KEYS_PER_TOKEN 1
#define ORC_VALUES_PER_CHANNEL 2

/* Row t (D elements, as stored: dequantized or verbatim) of one operand of
 * sequence/head bh in an n-token cache.
 *   per_token: groups are G channels of one token, planes
 *              codes[bh][tcap][D/G][W], meta[bh][tcap][D/G]; every token
 *              t >= ns is quantized unless a residual window R > 0 keeps
 *              [tq, n) in the ring (ring_values).
 *   otherwise: groups are one channel over G tokens, planes
 *              codes[bh][gcap][D][W], meta[bh][gcap][D]; tokens [ns, tq) are
 *              quantized and [tq, n) sit in ring slot t mod ring.
 *   t < ns:    sink row t. */
static void stored_row(int per_token, int ring_values, const uint32_t* codes,
                       const uint32_t* meta, const void* ring_buf,
                       const void* sink_buf, int dtype, size_t bh, int t, int n,
                       int D, int G, int bits, int R, int S, int gcap, int tcap,
                       double* row)
{
    int w = G * bits / 32, ncg = D / G, ring = R + G;
    int ns = n < S ? n : S;
    int tq = orc_quantized_end(n, G, R, S);
    if (t < ns) {
        for (int c = 0; c < D; ++c)
            row[c] = load_elem(sink_buf, dtype, (bh * S + t) * D + c);
    } else if (per_token && (!ring_values || t < tq)) {
        for (int cg = 0; cg < ncg; ++cg) {
            size_t tc = (bh * tcap + t) * ncg + cg;
            for (int j = 0; j < G; ++j)
                row[cg * G + j] = dequant(meta[tc],
                                          orc_code_at(codes + tc * w, j, bits));
        }
    } else if (!per_token && t < tq) {
        int g = t / G, j = t % G;
        for (int c = 0; c < D; ++c) {
            size_t gc = (bh * gcap + g) * D + c;
            row[c] = dequant(meta[gc], orc_code_at(codes + gc * w, j, bits));
        }
    } else {
        for (int c = 0; c < D; ++c)
            row[c] = load_elem(ring_buf, dtype, (bh * ring + t % ring) * D + c);
    }
}

/* Decode attention over a cache in any geometry (the bits of geom above),
 * rows [row_begin, row_end) as in orc_attend.  Keys per channel with R > 0
 * or S > 0 read the sink and ring as orc_attend does; the flipped
 * geometries are defined without windows (R = S = 0). */
int orc_attend_geometry(int nb, int hq, int hkv, int D, int G, int kbits,
                        int vbits, int geom, int R, int S, int gcap, int tcap,
                        double base, const uint32_t* k_codes,
                        const uint32_t* k_meta, const void* k_tail,
                        const void* k_sink, const uint32_t* v_codes,
                        const uint32_t* v_meta, const void* v_tail,
                        const void* v_sink, int dtype, const void* q, int n,
                        int row_begin, int row_end, double* out)
{
    if (n <= 0 || hkv <= 0 || hq % hkv != 0 || D % 2 != 0 || D % G != 0 ||
        n > tcap || n / G > gcap || row_begin < 0 || row_end > nb * hq ||
        geom < 0 || geom > 3 || R < 0 || R % G != 0 || S < 0 || S % G != 0 ||
        (geom != 0 && (R != 0 || S != 0)) || (S > 0 && (!k_sink || !v_sink)) ||
        ((R > 0 || (geom & ORC_VALUES_PER_CHANNEL)) && !v_tail))
        return -1;
    int kpt = (geom & ORC_KEYS_PER_TOKEN) != 0;
    int vpt = (geom & ORC_VALUES_PER_CHANNEL) == 0;
    double* score = (double*)malloc(sizeof(double) * (size_t)n);
    double* vals = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)D);
    if (!score || !vals || !qr || !kr) {
        free(score); free(vals); free(qr); free(kr);
        return -2;
    }
    int group = hq / hkv;
    for (int r = row_begin; r < row_end; ++r) {
        int b = r / hq, h = r % hq, kvh = h / group;
        size_t bh = (size_t)b * hkv + kvh;
        for (int c = 0; c < D; ++c)
            qr[c] = load_elem(q, dtype, (size_t)r * D + c);
        orc_rope(qr, D, (double)(n - 1), base);
        for (int t = 0; t < n; ++t) {
            stored_row(kpt, 0, k_codes, k_meta, k_tail, k_sink, dtype, bh, t, n,
                       D, G, kbits, R, S, gcap, tcap, kr);
            orc_rope(kr, D, (double)t, base);
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += qr[c] * kr[c];
            score[t] = dot / sqrt((double)D);
            stored_row(vpt, R > 0, v_codes, v_meta, v_tail, v_sink, dtype, bh, t,
                       n, D, G, vbits, R, S, gcap, tcap, vals + (size_t)t * D);
        }
        softmax_sum(score, vals, n, D, out + (size_t)(r - row_begin) * D);
    }
    free(score); free(vals); free(qr); free(kr);
    return 0;
}

/* Softmax weights (two-pass) of n scores, in place. */
static void softmax_weights(double* s, int n)
{
    double m = s[0], l = 0.0;
    for (int t = 1; t < n; ++t)
        if (s[t] > m) m = s[t];
    for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    for (int t = 0; t < n; ++t)
        s[t] /= l;
}

/* Error where it is consumed, per output row r in [row_begin, row_end)
 * (6 doubles each in rows_out), for a cache of n tokens holding the
 * unquantized keys k and values v ([nb][Hkv][n][D], the cache's dtype):
 *   [0] sum_t (ahat_t - a_t)^2      a = softmax(q'.RoPE(k_t)/sqrt(D)),
 *                                   ahat the same from the stored keys
 *   [1] |sum_t a_t vhat_t - sum_t a_t v_t|^2     (stored values, exact weights)
 *   [2] |sum_t a_t v_t|^2                        (the reference output)
 *   [3] |sum_t ahat_t vhat_t - sum_t a_t v_t|^2  (end to end)
 *   [4] sum_{t,c} (khat - k)^2 over the row's KV head (before the rotation)
 *   [5] sum_{t,c} (vhat - v)^2 over the row's KV head
 * "Stored" is what the cache holds: dequantized codes, or the verbatim tail,
 * ring and sink rows. */
int orc_error_metrics(int nb, int hq, int hkv, int D, int G, int kbits,
                      int vbits, int geom, int R, int S, int gcap, int tcap,
                      double base, const uint32_t* k_codes,
                      const uint32_t* k_meta, const void* k_tail,
                      const void* k_sink, const uint32_t* v_codes,
                      const uint32_t* v_meta, const void* v_tail,
                      const void* v_sink, int dtype, const void* k,
                      const void* v, const void* q, int n, int row_begin,
                      int row_end, double* rows_out)
{
    if (n <= 0 || hkv <= 0 || hq % hkv != 0 || D % 2 != 0 || D % G != 0 ||
        n > tcap || n / G > gcap || row_begin < 0 || row_end > nb * hq ||
        geom < 0 || geom > 3 || R < 0 || R % G != 0 || S < 0 || S % G != 0 ||
        (geom != 0 && (R != 0 || S != 0)) || (S > 0 && (!k_sink || !v_sink)) ||
        ((R > 0 || (geom & ORC_VALUES_PER_CHANNEL)) && !v_tail))
        return -1;
    int kpt = (geom & ORC_KEYS_PER_TOKEN) != 0;
    int vpt = (geom & ORC_VALUES_PER_CHANNEL) == 0;
    size_t nd = (size_t)n * D;
    double* a = (double*)malloc(sizeof(double) * (size_t)n);
    double* ah = (double*)malloc(sizeof(double) * (size_t)n);
    double* kx = (double*)malloc(sizeof(double) * nd);
    double* kh = (double*)malloc(sizeof(double) * nd);
    double* vx = (double*)malloc(sizeof(double) * nd);
    double* vh = (double*)malloc(sizeof(double) * nd);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* o = (double*)malloc(sizeof(double) * (size_t)D * 3);
    if (!a || !ah || !kx || !kh || !vx || !vh || !qr || !o) {
        free(a); free(ah); free(kx); free(kh); free(vx); free(vh); free(qr); free(o);
        return -2;
    }
    int group = hq / hkv;
    for (int r = row_begin; r < row_end; ++r) {
        int b = r / hq, h = r % hq, kvh = h / group;
        size_t bh = (size_t)b * hkv + kvh;
        double* m = rows_out + (size_t)(r - row_begin) * 6;
        for (int i = 0; i < 6; ++i)
            m[i] = 0.0;
        for (int t = 0; t < n; ++t) {
            stored_row(kpt, 0, k_codes, k_meta, k_tail, k_sink, dtype, bh, t, n,
                       D, G, kbits, R, S, gcap, tcap, kh + (size_t)t * D);
            stored_row(vpt, R > 0, v_codes, v_meta, v_tail, v_sink, dtype, bh, t,
                       n, D, G, vbits, R, S, gcap, tcap, vh + (size_t)t * D);
            for (int c = 0; c < D; ++c) {
                size_t i = (size_t)t * D + c;
                kx[i] = load_elem(k, dtype, (bh * n + t) * D + c);
                vx[i] = load_elem(v, dtype, (bh * n + t) * D + c);
                m[4] += (kh[i] - kx[i]) * (kh[i] - kx[i]);
                m[5] += (vh[i] - vx[i]) * (vh[i] - vx[i]);
            }
        }
        for (int c = 0; c < D; ++c)
            qr[c] = load_elem(q, dtype, (size_t)r * D + c);
        orc_rope(qr, D, (double)(n - 1), base);
        for (int t = 0; t < n; ++t) {
            orc_rope(kx + (size_t)t * D, D, (double)t, base);
            orc_rope(kh + (size_t)t * D, D, (double)t, base);
            double d0 = 0.0, d1 = 0.0;
            for (int c = 0; c < D; ++c) {
                d0 += qr[c] * kx[(size_t)t * D + c];
                d1 += qr[c] * kh[(size_t)t * D + c];
            }
            a[t] = d0 / sqrt((double)D);
            ah[t] = d1 / sqrt((double)D);
        }
        softmax_weights(a, n);
        softmax_weights(ah, n);
        for (int i = 0; i < 3 * D; ++i)
            o[i] = 0.0;
        for (int t = 0; t < n; ++t) {
            m[0] += (ah[t] - a[t]) * (ah[t] - a[t]);
            for (int c = 0; c < D; ++c) {
                size_t i = (size_t)t * D + c;
                o[c] += a[t] * vx[i];          /* reference */
                o[D + c] += a[t] * vh[i];      /* stored values */
                o[2 * D + c] += ah[t] * vh[i]; /* end to end */
            }
        }
        for (int c = 0; c < D; ++c) {
            m[1] += (o[D + c] - o[c]) * (o[D + c] - o[c]);
            m[2] += o[c] * o[c];
            m[3] += (o[2 * D + c] - o[c]) * (o[2 * D + c] - o[c]);
        }
    }
    free(a); free(ah); free(kx); free(kh); free(vx); free(vh); free(qr); free(o);
    return 0;
}

/* ------------------------------------------------------------- FP8 E4M3 */

/* Value of an OCP FP8 E4M3 byte: sign, exponent e (bias 7), mantissa m:
 * e = 0 is subnormal, m * 2^-9; e = 15 with m = 7 is NaN. */
double orc_fp8_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 byte to x (finite), ties to the even mantissa, magnitudes at
 * or above 448 saturate to 448. */
uint8_t orc_fp8_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7E;
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    if (e < -6)
        e = -6;             /* subnormal steps are 2^-9 like the lowest binade */
    double q = rint(ldexp(a, 3 - e));   /* multiples of 2^(e-3), ties to even */
    if (a < ldexp(1.0, -6)) {           /* subnormal: code = q (q = 8 is 2^-6) */
        return sign | (uint8_t)q;
    }
    if (q >= 16.0) {        /* rounded up into the next binade */
        q = 8.0;
        e += 1;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* Byte of token j (< 32), channel c inside a group block of D * 32 bytes:
 * the logical, channel-major order. */
static size_t fp8_offset(int c, int j)
{
    return (size_t)c * 32 + (size_t)j;
}

/* FP8 planes for T tokens of x[nb][Hkv][T][D] (keys or values), group g of
 * sequence/head bh in block bh * gcap + g (G must be 32); bytes of a partly
 * filled group past T are 0. */
int orc_quantize_fp8(const void* x, int dtype, int nb, int hkv, int T, int D,
                     int G, int gcap, uint8_t* planes)
{
    if (G != 32 || T < 0 || (T + G - 1) / G > gcap || D % 2 != 0)
        return -1;
    int ng = (T + G - 1) / G;
    for (int b = 0; b < nb; ++b)
        for (int h = 0; h < hkv; ++h) {
            size_t bh = (size_t)b * hkv + h;
            for (int g = 0; g < ng; ++g)
                for (int c = 0; c < D; ++c)
                    for (int j = 0; j < G; ++j) {
                        int t = g * G + j;
                        size_t o = (bh * gcap + g) * D * G + fp8_offset(c, j);
                        planes[o] = t < T ? orc_fp8_encode(load_elem(
                                                x, dtype, (bh * T + t) * D + c))
                                          : 0;
                    }
        }
    return 0;
}

/* Decode attention over FP8 planes (the layout above) for rows
 * [row_begin, row_end): keys decoded and rotated to position t, the query
 * to n-1, scores / sqrt(D), softmax-weighted sum of the decoded values. */
int orc_attend_fp8(int nb, int hq, int hkv, int D, int G, int gcap, double base,
                   const uint8_t* k8, const uint8_t* v8, int dtype,
                   const void* q, int n, int row_begin, int row_end,
                   double* out)
{
    if (n <= 0 || hkv <= 0 || hq % hkv != 0 || D % 2 != 0 || G != 32 ||
        (n + G - 1) / G > gcap || row_begin < 0 || row_end > nb * hq)
        return -1;
    double* score = (double*)malloc(sizeof(double) * (size_t)n);
    double* vals = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)D);
    if (!score || !vals || !qr || !kr) {
        free(score); free(vals); free(qr); free(kr);
        return -2;
    }
    int group = hq / hkv;
    for (int r = row_begin; r < row_end; ++r) {
        int b = r / hq, h = r % hq, kvh = h / group;
        size_t bh = (size_t)b * hkv + kvh;
        for (int c = 0; c < D; ++c)
            qr[c] = load_elem(q, dtype, (size_t)r * D + c);
        orc_rope(qr, D, (double)(n - 1), base);
        for (int t = 0; t < n; ++t) {
            for (int c = 0; c < D; ++c) {
                size_t o = (bh * gcap + t / G) * D * G + fp8_offset(c, t % G);
                kr[c] = orc_fp8_decode(k8[o]);
                vals[(size_t)t * D + c] = orc_fp8_decode(v8[o]);
            }
            orc_rope(kr, D, (double)t, base);
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += qr[c] * kr[c];
            score[t] = dot / sqrt((double)D);
        }
        softmax_sum(score, vals, n, D, out + (size_t)(r - row_begin) * D);
    }
    free(score); free(vals); free(qr); free(kr);
    return 0;
}
