// Driver for the GPU library's host code (kvq_host.cpp) built for the CPU
// under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py).  The HIP runtime calls and the kernel
// launchers are replaced by stubs: "device" memory is host memory, a copy is
// memcpy, and each launcher, instead of enqueuing a kernel, reads the first
// and last element of every plane and buffer the kernel would touch, with
// extents computed from the plane layout.  A workspace of exactly
// kvq_workspace_bytes bytes then makes any disagreement between the layout
// arithmetic, the planes handed to the kernels and the buffers' sizes an
// out-of-bounds report.  Every entry point runs, with its error paths.
//
// Test infrastructure only.
#include "kvq.h"
#include "kvq_internal.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

// ------------------------------------------------------------ HIP stubs --

static int g_launches = 0;

extern "C" {
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind)
{
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}
hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int)
{
    std::memset(prop, 0, sizeof(*prop));
    prop->multiProcessorCount = 256;
    return hipSuccess;
}
}

namespace kvqi {

static unsigned char* g_scratch = nullptr;

hipError_t static_scratch(int, void** out)
{
    if (!g_scratch)
        g_scratch = static_cast<unsigned char*>(std::aligned_alloc(256, kStaticScratchBytes));
    *out = g_scratch;
    return hipSuccess;
}

// First and last byte of [p, p + bytes) (nothing when empty).
static volatile unsigned char g_sink;
static void touch(const void* p, size_t bytes)
{
    if (bytes == 0)
        return;
    const unsigned char* c = static_cast<const unsigned char*>(p);
    g_sink = c[0];
    g_sink = c[bytes - 1];
}

static size_t esz(const Planes& p) { return p.dtype == KVQ_F16 ? 2 : 4; }

// Every plane at its full extent, from the layout's formulas.
static void touch_planes(const Planes& p)
{
    const size_t nbh = (size_t)p.nb * p.hkv, D = p.D, G = kGroup;
    const size_t wk = G * p.kbits / 32, wv = G * p.vbits / 32;
    if (p.format == kFormatFp8) {
        touch(p.k_codes, nbh * p.gcap * D * G);
        touch(p.v_codes, nbh * p.gcap * D * G);
    } else {
        const bool kpt = (p.geometry & kKeysPerToken) != 0;
        const bool vpc = (p.geometry & kValuesPerChannel) != 0;
        touch(p.k_codes, (kpt ? nbh * p.tcap * (D / G) : nbh * p.gcap * D) * wk * 4);
        touch(p.k_meta, (kpt ? nbh * p.tcap * (D / G) : nbh * p.gcap * D) * 4);
        touch(p.v_codes, (vpc ? nbh * p.gcap * D : nbh * p.tcap * (D / G)) * wv * 4);
        touch(p.v_meta, (vpc ? nbh * p.gcap * D : nbh * p.tcap * (D / G)) * 4);
        touch(p.k_tail, nbh * p.ring * D * esz(p));
        if (p.residual > 0 || vpc)
            touch(p.v_tail, nbh * p.ring * D * esz(p));
        touch(p.k_sink, nbh * p.sink * D * esz(p));
        touch(p.v_sink, nbh * p.sink * D * esz(p));
    }
    touch(p.rope_group, (size_t)p.gcap * (D / 2) * sizeof(float2));
    touch(p.rope_offset, G * (D / 2) * sizeof(float2));
}

static void touch_tokens(const Planes& p, const void* x, int n)
{
    touch(x, (size_t)p.nb * p.hkv * n * p.D * esz(p));
}

static void touch_attend(const Planes& p, const void* q, float* out, int splits)
{
    const size_t rows = (size_t)p.nb * p.hq;
    touch(q, rows * p.D * esz(p));
    touch(out, rows * p.D * sizeof(float));
    if (splits > 1) {
        if (splits > p.max_splits)
            std::abort();
        touch(p.partials, rows * p.max_splits * (p.D + 2) * sizeof(float));
    }
}

hipError_t launch_quantize_prefill(const Planes& p, const void* k, const void* v, int n,
                                   hipStream_t)
{
    ++g_launches;
    touch_planes(p);
    touch_tokens(p, k, n);
    touch_tokens(p, v, n);
    return hipSuccess;
}

hipError_t launch_append(const Planes& p, const void* k, const void* v, int, hipStream_t)
{
    ++g_launches;
    touch_planes(p);
    touch_tokens(p, k, 1);
    touch_tokens(p, v, 1);
    return hipSuccess;
}

static hipError_t attend(const Planes& p, const void* q, float* out, int splits,
                         const void* k_new, const void* v_new)
{
    ++g_launches;
    touch_planes(p);
    touch_attend(p, q, out, splits);
    if (k_new) {
        touch_tokens(p, k_new, 1);
        touch_tokens(p, v_new, 1);
    }
    return hipSuccess;
}

hipError_t launch_attend_d64(const Planes& p, const void* q, float* out, int, int splits, int,
                             const void* k_new, const void* v_new, hipStream_t)
{
    return attend(p, q, out, splits, k_new, v_new);
}

hipError_t launch_attend_d128(const Planes& p, const void* q, float* out, int, int splits, int,
                              const void* k_new, const void* v_new, hipStream_t)
{
    return attend(p, q, out, splits, k_new, v_new);
}

hipError_t launch_attend_geometry(const Planes& p, const void* q, float* out, int, int splits,
                                  hipStream_t)
{
    return attend(p, q, out, splits, nullptr, nullptr);
}

hipError_t launch_fp8_prefill(const Planes& p, const void* k, const void* v, int n, hipStream_t s)
{
    return launch_quantize_prefill(p, k, v, n, s);
}

hipError_t launch_fp8_append(const Planes& p, const void* k, const void* v, int n, hipStream_t s)
{
    return launch_append(p, k, v, n, s);
}

hipError_t launch_attend_fp8(const Planes& p, const void* q, float* out, int, int splits,
                             hipStream_t)
{
    return attend(p, q, out, splits, nullptr, nullptr);
}

hipError_t launch_error_metrics(const Planes& p, const void* k, const void* v, const void* q,
                                double* metrics, int n, hipStream_t)
{
    ++g_launches;
    touch_planes(p);
    touch_tokens(p, k, n);
    touch_tokens(p, v, n);
    touch(q, (size_t)p.nb * p.hq * p.D * esz(p));
    touch(metrics, 5 * sizeof(double));
    return hipSuccess;
}

}  // namespace kvqi

// --------------------------------------------------------------- driver --

static int g_fail = 0;

static void expect(int got, int want, const char* what, int line)
{
    if (got != want) {
        std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
        ++g_fail;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static kvq_config base_cfg()
{
    kvq_config c;
    std::memset(&c, 0, sizeof c);
    c.batch = 2;
    c.q_heads = 4;
    c.kv_heads = 4;
    c.head_dim = 64;
    c.max_tokens = 100;
    c.group = 32;
    c.key_bits = 2;
    c.value_bits = 2;
    c.dtype = KVQ_F16;
    c.rope_base = 10000.0f;
    c.format = KVQ_FORMAT_INT;
    return c;
}

static std::vector<unsigned char> host_buf(size_t bytes) { return std::vector<unsigned char>(bytes); }

// A whole life cycle on one configuration, with its state and capacity errors.
static void life_cycle(const kvq_config& c, int prompt)
{
    const size_t ws_bytes = kvq_workspace_bytes(&c);
    if (ws_bytes == 0) {
        std::fprintf(stderr, "configuration rejected\n");
        ++g_fail;
        return;
    }
    kvq_layout L;
    EXPECT(kvq_layout_for(&c, &L), KVQ_OK);
    if (L.total_bytes != ws_bytes)
        ++g_fail;
    // exactly the workspace size (a multiple of 256), so ASan sees its end
    void* ws = std::aligned_alloc(256, ws_bytes);
    kvq_t* h = nullptr;
    EXPECT(kvq_create(&c, ws, ws_bytes - 256, &h), KVQ_ERR_WORKSPACE);
    EXPECT(kvq_create(&c, static_cast<char*>(ws) + 16, ws_bytes, &h), KVQ_ERR_WORKSPACE);
    EXPECT(kvq_create(&c, ws, ws_bytes, &h), KVQ_OK);
    if (!h) {
        std::free(ws);
        return;
    }
    const size_t esz = c.dtype == KVQ_F16 ? 2 : 4;
    const size_t tok = (size_t)c.batch * c.kv_heads * c.head_dim * esz;
    auto k = host_buf(tok * c.max_tokens), v = host_buf(tok * c.max_tokens);
    auto q = host_buf((size_t)c.batch * c.q_heads * c.head_dim * esz);
    std::vector<float> out((size_t)c.batch * c.q_heads * c.head_dim);
    std::vector<double> met(5);
    EXPECT(kvq_attend_decode(h, q.data(), out.data(), nullptr), KVQ_ERR_STATE);
    EXPECT(kvq_error_metrics(h, k.data(), v.data(), q.data(), met.data(), nullptr),
           KVQ_ERR_STATE);
    EXPECT(kvq_quantize_prefill(h, k.data(), v.data(), c.max_tokens + 1, nullptr),
           KVQ_ERR_CAPACITY);
    EXPECT(kvq_quantize_prefill(h, nullptr, v.data(), prompt, nullptr),
           prompt > 0 ? KVQ_ERR_ARG : KVQ_OK);
    auto kp = host_buf(tok * (prompt > 0 ? prompt : 1)), vp = host_buf(tok * (prompt > 0 ? prompt : 1));
    EXPECT(kvq_quantize_prefill(h, kp.data(), vp.data(), prompt, nullptr), KVQ_OK);
    EXPECT(kvq_length(h), prompt);
    if (prompt > 0)
        EXPECT(kvq_quantize_prefill(h, kp.data(), vp.data(), prompt, nullptr), KVQ_ERR_STATE);
    auto k1 = host_buf(tok), v1 = host_buf(tok);
    int n = prompt;
    while (n < c.max_tokens) {
        int st;
        switch (n % 3) {
        case 0: st = kvq_append_attend(h, k1.data(), v1.data(), q.data(), out.data(), nullptr); break;
        case 1: st = kvq_append_token(h, k1.data(), v1.data(), nullptr); break;
        default:
            st = kvq_append_attend_static(h, k1.data(), v1.data(), q.data(), out.data(), nullptr);
            break;
        }
        if (st == KVQ_ERR_SCRATCH) {  // too many splits for the static scratch: plain step
            st = kvq_append_attend(h, k1.data(), v1.data(), q.data(), out.data(), nullptr);
        }
        EXPECT(st, KVQ_OK);
        if (st != KVQ_OK)
            break;
        ++n;
        EXPECT(kvq_attend_decode(h, q.data(), out.data(), nullptr), KVQ_OK);
    }
    EXPECT(kvq_append_token(h, k1.data(), v1.data(), nullptr), KVQ_ERR_CAPACITY);
    EXPECT(kvq_append_attend(h, k1.data(), v1.data(), q.data(), out.data(), nullptr),
           KVQ_ERR_CAPACITY);
    EXPECT(kvq_error_metrics(h, k.data(), v.data(), q.data(), met.data(), nullptr),
           c.format == KVQ_FORMAT_INT ? KVQ_OK : KVQ_ERR_UNSUPPORTED);
    kvq_layout got;
    EXPECT(kvq_get_layout(h, &got), KVQ_OK);
    EXPECT(kvq_destroy(h), KVQ_OK);
    std::free(ws);
}

int main()
{
    // argument and configuration errors (pure host)
    EXPECT(kvq_layout_for(nullptr, nullptr), KVQ_ERR_ARG);
    kvq_layout L;
    kvq_config c = base_cfg();
    c.head_dim = 96;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_UNSUPPORTED);
    c = base_cfg();
    c.q_heads = 6;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_ARG);
    c = base_cfg();
    c.max_tokens = (1 << 24) + 1;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_UNSUPPORTED);
    c = base_cfg();
    c.batch = 1 << 20;
    c.q_heads = c.kv_heads = 64;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_UNSUPPORTED);
    c = base_cfg();
    c.residual = 33;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_UNSUPPORTED);
    c = base_cfg();
    c.format = KVQ_FORMAT_FP8_E4M3;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_UNSUPPORTED);
    c = base_cfg();
    c.rope_base = 1.0f;
    EXPECT(kvq_layout_for(&c, &L), KVQ_ERR_ARG);
    EXPECT(kvq_destroy(nullptr), KVQ_ERR_ARG);
    EXPECT(kvq_length(nullptr), -1);
    if (!kvq_strerror(KVQ_ERR_HIP) || !kvq_strerror(12345))
        ++g_fail;

    // life cycles over the supported space
    for (int dtype : {KVQ_F16, KVQ_F32})
        for (int D : {64, 128})
            for (int qpk : {1, 2, 4, 8}) {
                c = base_cfg();
                c.dtype = dtype;
                c.head_dim = D;
                c.q_heads = 2 * qpk;
                c.kv_heads = 2;
                life_cycle(c, 45);
            }
    for (int kb : {2, 4, 8})
        for (int vb : {2, 4, 8}) {
            c = base_cfg();
            c.key_bits = kb;
            c.value_bits = vb;
            life_cycle(c, 0);
        }
    c = base_cfg();
    c.residual = 64;
    c.max_tokens = 200;
    life_cycle(c, 70);
    c.sink = 32;
    life_cycle(c, 10);
    for (int geom = 1; geom <= 3; ++geom) {
        c = base_cfg();
        c.geometry = geom;
        life_cycle(c, 33);
    }
    c = base_cfg();
    c.key_bits = c.value_bits = 8;
    c.format = KVQ_FORMAT_FP8_E4M3;
    life_cycle(c, 31);
    c = base_cfg();  // one sequence, long context: many splits
    c.batch = 1;
    c.q_heads = c.kv_heads = 1;
    c.max_tokens = 4096;
    life_cycle(c, 4000);
    setenv("KVQ_SYNC", "1", 1);  // the debug-sync path
    c = base_cfg();
    life_cycle(c, 50);
    unsetenv("KVQ_SYNC");

    if (g_launches == 0)
        ++g_fail;
    if (g_fail) {
        std::fprintf(stderr, "%d failures\n", g_fail);
        return 1;
    }
    std::printf("ok (%d launches)\n", g_launches);
    std::free(kvqi::g_scratch);
    return 0;
}
