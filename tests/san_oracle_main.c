/* Driver that runs every entry point of the C oracle (oracle/oracle.c) on
 * small caches, for builds under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (tests/test_sanitizers.py).  Every buffer is allocated at exactly
 * the size the oracle's plane layout needs, so an access past a plane's end
 * is reported.  Exit status 0 and no sanitizer report is the pass; results
 * are checked elsewhere (the oracle's own tests).
 *
 * Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double x);
int orc_quant_group(const double* x, int n, int bits, uint8_t* codes, uint16_t* s16_out,
                    uint16_t* z16_out);
void orc_pack(const uint8_t* codes, int n, int bits, uint32_t* words);
int orc_code_at(const uint32_t* words, int j, int bits);
void orc_unpack(const uint32_t* words, int n, int bits, uint8_t* codes);
int orc_quantized_end(int n, int G, int R, int S);
int orc_quantize_keys(const void* k, int dtype, int nb, int hkv, int T, int D, int G, int bits,
                      int R, int S, int gcap, uint32_t* k_codes, uint32_t* k_meta, void* k_tail,
                      void* k_sink);
int orc_quantize_values(const void* v, int dtype, int nb, int hkv, int T, int D, int G, int bits,
                        int R, int S, int tcap, uint32_t* v_codes, uint32_t* v_meta,
                        void* v_tail, void* v_sink);
void orc_rope(double* u, int D, double p, double base);
int orc_attend(int nb, int hq, int hkv, int D, int G, int kbits, int vbits, int R, int S,
               int gcap, int tcap, double base, const uint32_t* k_codes,
               const uint32_t* k_meta, const void* k_tail, const void* k_sink,
               const uint32_t* v_codes, const uint32_t* v_meta, const void* v_tail,
               const void* v_sink, int dtype, const void* q, int n, int row_begin,
               int row_end, double* out);
int orc_attend_dense(int nb, int hq, int hkv, int D, double base, const void* k, const void* v,
                     int dtype, const void* q, int n, int row_begin, int row_end, double* out);
int orc_attend_geometry(int nb, int hq, int hkv, int D, int G, int kbits, int vbits, int geom,
                        int R, int S, int gcap, int tcap, double base, const uint32_t* k_codes,
                        const uint32_t* k_meta, const void* k_tail, const void* k_sink,
                        const uint32_t* v_codes, const uint32_t* v_meta, const void* v_tail,
                        const void* v_sink, int dtype, const void* q, int n, int row_begin,
                        int row_end, double* out);
int orc_error_metrics(int nb, int hq, int hkv, int D, int G, int kbits, int vbits, int geom,
                      int R, int S, int gcap, int tcap, double base, const uint32_t* k_codes,
                      const uint32_t* k_meta, const void* k_tail, const void* k_sink,
                      const uint32_t* v_codes, const uint32_t* v_meta, const void* v_tail,
                      const void* v_sink, int dtype, const void* k, const void* v,
                      const void* q, int n, int row_begin, int row_end, double* rows_out);
double orc_fp8_decode(uint8_t b);
uint8_t orc_fp8_encode(double x);
int orc_quantize_fp8(const void* x, int dtype, int nb, int hkv, int T, int D, int G, int gcap,
                     uint8_t* planes);
int orc_attend_fp8(int nb, int hq, int hkv, int D, int G, int gcap, double base,
                   const uint8_t* k8, const uint8_t* v8, int dtype, const void* q, int n,
                   int row_begin, int row_end, double* out);

enum { G = 32 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64, then a uniform in [-1, 1) */
static double uniform(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1p-52 - 1.0;
}

static void* xmalloc(size_t bytes)
{
    void* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    memset(p, 0, bytes ? bytes : 1);
    return p;
}

/* n elements of the given dtype (0 binary16, 1 fp32), values scale * U(-1, 1)
 * with every 7th channel scaled by 20 (outlier channels) */
static void* make_input(int dtype, size_t n, int D, double scale)
{
    void* p = xmalloc(n * (dtype == 0 ? 2 : 4));
    for (size_t i = 0; i < n; ++i) {
        double x = scale * uniform() * ((i % (size_t)D) % 7 == 3 ? 20.0 : 1.0);
        if (dtype == 0)
            ((uint16_t*)p)[i] = orc_double_to_half(x);
        else
            ((float*)p)[i] = (float)x;
    }
    return p;
}

static int failures = 0;

static void expect_ok(int rc, const char* what)
{
    if (rc != 0) {
        fprintf(stderr, "%s returned %d\n", what, rc);
        ++failures;
    }
}

static void run_cache(int dtype, int kbits, int vbits, int R, int S, int T, int cap)
{
    const int nb = 2, hkv = 2, hq = 4, D = 64;
    const int gcap = (cap + G - 1) / G, tcap = gcap * G, ring = R + G;
    const int wk = G * kbits / 32, wv = G * vbits / 32;
    const size_t esz = dtype == 0 ? 2 : 4, nbh = (size_t)nb * hkv, rows = (size_t)nb * hq;
    void* k = make_input(dtype, nbh * T * D, D, 1.0);
    void* v = make_input(dtype, nbh * T * D, D, 0.5);
    void* q = make_input(dtype, rows * D, D, 1.0);
    uint32_t* kc = xmalloc(nbh * gcap * D * wk * 4);
    uint32_t* km = xmalloc(nbh * gcap * D * 4);
    void* kt = xmalloc(nbh * ring * D * esz);
    void* ks = S > 0 ? xmalloc(nbh * S * D * esz) : NULL;
    uint32_t* vc = xmalloc(nbh * tcap * (D / G) * wv * 4);
    uint32_t* vm = xmalloc(nbh * tcap * (D / G) * 4);
    void* vt = R > 0 ? xmalloc(nbh * ring * D * esz) : NULL;
    void* vs = S > 0 ? xmalloc(nbh * S * D * esz) : NULL;
    double* out = xmalloc(rows * D * sizeof(double));
    double* met = xmalloc(rows * 6 * sizeof(double));
    expect_ok(orc_quantize_keys(k, dtype, nb, hkv, T, D, G, kbits, R, S, gcap, kc, km, kt, ks),
              "orc_quantize_keys");
    expect_ok(orc_quantize_values(v, dtype, nb, hkv, T, D, G, vbits, R, S, tcap, vc, vm, vt, vs),
              "orc_quantize_values");
    for (int n = 1; n <= T; n += (n < 40 ? 13 : T - n > 0 ? T - n : 1)) {
        expect_ok(orc_attend(nb, hq, hkv, D, G, kbits, vbits, R, S, gcap, tcap, 10000.0, kc, km,
                             kt, ks, vc, vm, vt, vs, dtype, q, n, 0, (int)rows, out),
                  "orc_attend");
        if (n == T)
            expect_ok(orc_attend_geometry(nb, hq, hkv, D, G, kbits, vbits, 0, R, S, gcap, tcap,
                                          10000.0, kc, km, kt, ks, vc, vm, vt, vs, dtype, q, n,
                                          1, (int)rows - 1, out),
                      "orc_attend_geometry");
    }
    expect_ok(orc_error_metrics(nb, hq, hkv, D, G, kbits, vbits, 0, R, S, gcap, tcap, 10000.0, kc,
                                km, kt, ks, vc, vm, vt, vs, dtype, k, v, q, T, 0, (int)rows, met),
              "orc_error_metrics");
    expect_ok(orc_attend_dense(nb, hq, hkv, D, 10000.0, k, v, dtype, q, T, 0, (int)rows, out),
              "orc_attend_dense");
    free(kc); free(km); free(kt); free(ks); free(vc); free(vm); free(vt); free(vs);

    if (R == 0 && S == 0) {
        /* the geometry ablation: keys per token (value layout, key tail of G
         * slots unused), values per channel (key layout with a G-slot tail) */
        for (int geom = 1; geom <= 3; ++geom) {
            const int kpt = geom & 1, vpc = geom & 2;
            uint32_t* gkc = xmalloc(kpt ? nbh * tcap * (D / G) * wk * 4 : nbh * gcap * D * wk * 4);
            uint32_t* gkm = xmalloc(kpt ? nbh * tcap * (D / G) * 4 : nbh * gcap * D * 4);
            void* gkt = xmalloc(nbh * G * D * esz);
            uint32_t* gvc = xmalloc(vpc ? nbh * gcap * D * wv * 4 : nbh * tcap * (D / G) * wv * 4);
            uint32_t* gvm = xmalloc(vpc ? nbh * gcap * D * 4 : nbh * tcap * (D / G) * 4);
            void* gvt = vpc ? xmalloc(nbh * G * D * esz) : NULL;
            if (kpt)
                expect_ok(orc_quantize_values(k, dtype, nb, hkv, T, D, G, kbits, 0, 0, tcap, gkc,
                                              gkm, NULL, NULL), "keys per token");
            else
                expect_ok(orc_quantize_keys(k, dtype, nb, hkv, T, D, G, kbits, 0, 0, gcap, gkc,
                                            gkm, gkt, NULL), "keys per channel");
            if (vpc)
                expect_ok(orc_quantize_keys(v, dtype, nb, hkv, T, D, G, vbits, 0, 0, gcap, gvc,
                                            gvm, gvt, NULL), "values per channel");
            else
                expect_ok(orc_quantize_values(v, dtype, nb, hkv, T, D, G, vbits, 0, 0, tcap, gvc,
                                              gvm, NULL, NULL), "values per token");
            expect_ok(orc_attend_geometry(nb, hq, hkv, D, G, kbits, vbits, geom, 0, 0, gcap, tcap,
                                          10000.0, gkc, gkm, gkt, NULL, gvc, gvm, gvt, NULL,
                                          dtype, q, T, 0, (int)rows, out),
                      "orc_attend_geometry");
            expect_ok(orc_error_metrics(nb, hq, hkv, D, G, kbits, vbits, geom, 0, 0, gcap, tcap,
                                        10000.0, gkc, gkm, gkt, NULL, gvc, gvm, gvt, NULL, dtype,
                                        k, v, q, T, 0, (int)rows, met),
                      "orc_error_metrics (geometry)");
            free(gkc); free(gkm); free(gkt); free(gvc); free(gvm); free(gvt);
        }
        if (kbits == 8 && vbits == 8) {
            uint8_t* k8 = xmalloc(nbh * gcap * D * G);
            uint8_t* v8 = xmalloc(nbh * gcap * D * G);
            expect_ok(orc_quantize_fp8(k, dtype, nb, hkv, T, D, G, gcap, k8), "orc_quantize_fp8");
            expect_ok(orc_quantize_fp8(v, dtype, nb, hkv, T, D, G, gcap, v8), "orc_quantize_fp8");
            expect_ok(orc_attend_fp8(nb, hq, hkv, D, G, gcap, 10000.0, k8, v8, dtype, q, T, 0,
                                     (int)rows, out),
                      "orc_attend_fp8");
            free(k8); free(v8);
        }
    }
    free(k); free(v); free(q); free(out); free(met);
}

int main(void)
{
    /* scalar helpers over their whole domains */
    for (uint32_t h = 0; h < 0x10000u; ++h) {
        const double x = orc_half_to_double((uint16_t)h);
        if (x == x && orc_double_to_half(x) != (uint16_t)h && (h & 0x7fffu) != 0)
            ++failures;
    }
    for (int b = 0; b < 256; ++b) {
        const double x = orc_fp8_decode((uint8_t)b);
        if (x == x)
            (void)orc_fp8_encode(x);
    }
    double u[128];
    for (int i = 0; i < 128; ++i)
        u[i] = uniform();
    orc_rope(u, 128, 4095.0, 10000.0);

    /* one group at every width, incl. constant and tiny-range groups */
    for (int bits = 2; bits <= 8; bits *= 2) {
        for (int kind = 0; kind < 4; ++kind) {
            double x[G];
            uint8_t codes[G], back[G];
            uint32_t words[8];
            uint16_t s16, z16;
            for (int j = 0; j < G; ++j)
                x[j] = kind == 0 ? uniform() : kind == 1 ? 1.25 : kind == 2 ? j * 0x1p-24
                                                                           : 1e4 * uniform();
            expect_ok(orc_quant_group(x, G, bits, codes, &s16, &z16), "orc_quant_group");
            memset(words, 0, sizeof words);
            orc_pack(codes, G, bits, words);
            orc_unpack(words, G, bits, back);
            for (int j = 0; j < G; ++j)
                if (back[j] != codes[j] || orc_code_at(words, j, bits) != codes[j])
                    ++failures;
        }
    }
    for (int n = 0; n < 200; ++n)
        (void)orc_quantized_end(n, G, 64, 32);

    /* whole caches: both element types, every width pair, windows */
    static const int widths[][2] = {{2, 2}, {4, 4}, {8, 8}, {2, 8}, {8, 4}};
    for (int dtype = 0; dtype <= 1; ++dtype)
        for (int w = 0; w < 5; ++w) {
            run_cache(dtype, widths[w][0], widths[w][1], 0, 0, 70, 96);
            run_cache(dtype, widths[w][0], widths[w][1], 0, 0, 20, 20);
        }
    run_cache(0, 2, 2, 32, 0, 130, 160);
    run_cache(0, 4, 2, 0, 32, 100, 128);
    run_cache(1, 2, 4, 32, 32, 140, 160);
    run_cache(0, 2, 2, 32, 32, 20, 64);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
