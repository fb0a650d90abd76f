// kvq_host.cpp -- the C ABI declared in include/kvq.h: configuration checks,
// workspace layout, the host-side length counter, rotary tables and kernel
// dispatch.  Every check runs before anything is enqueued.
#include "kvq.h"
#include "kvq_internal.h"

#include <cmath>
#include <cstdlib>
#include <new>
#include <vector>

struct kvq {
    kvq_config cfg;
    kvq_layout layout;
    char* ws;
    int32_t n;
    int32_t cus;            // compute units of the device the handle was made on
    int32_t force_splits;   // tuning overrides (KVQ_ATTEND_SPLITS / KVQ_ATTEND_WAVES), 0 = auto
    int32_t force_waves;
    int32_t sync;           // KVQ_SYNC=1: each call waits for its work and checks for a fault
    float* scratch;         // the library's static device scratch on the handle's device
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kTargetBlocks = 1024;  // attend blocks wanted per launch
constexpr int kMaxSplits = 256;
constexpr int kMaxResidual = 1024;  // tokens of a full-precision window (residual, sink)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_config(const kvq_config* c)
{
    if (!c)
        return KVQ_ERR_ARG;
    if (c->batch < 1 || c->q_heads < 1 || c->kv_heads < 1 || c->head_dim < 1 ||
        c->max_tokens < 1 || c->group < 1 || c->key_bits < 1 || c->value_bits < 1 ||
        !(c->rope_base > 1.0f) || !std::isfinite(c->rope_base) || c->q_heads % c->kv_heads != 0 ||
        (c->dtype != KVQ_F16 && c->dtype != KVQ_F32) || c->residual < 0 || c->sink < 0 ||
        c->geometry < 0 || c->geometry > (KVQ_KEYS_PER_TOKEN | KVQ_VALUES_PER_CHANNEL) ||
        (c->format != KVQ_FORMAT_INT && c->format != KVQ_FORMAT_FP8_E4M3))
        return KVQ_ERR_ARG;
    const int qpk = c->q_heads / c->kv_heads;
    if (c->group != kvqi::kGroup || (c->head_dim != 64 && c->head_dim != 128) ||
        (c->key_bits != 2 && c->key_bits != 4 && c->key_bits != 8) ||
        (c->value_bits != 2 && c->value_bits != 4 && c->value_bits != 8) ||
        (qpk != 1 && qpk != 2 && qpk != 4 && qpk != 8) || c->residual % kvqi::kGroup != 0 ||
        c->residual > kMaxResidual || c->sink % kvqi::kGroup != 0 || c->sink > kMaxResidual ||
        (c->geometry != 0 && (c->residual != 0 || c->sink != 0)) ||
        (c->format == KVQ_FORMAT_FP8_E4M3 &&
         (c->key_bits != 8 || c->value_bits != 8 || c->residual != 0 || c->sink != 0 ||
          c->geometry != 0)))
        return KVQ_ERR_UNSUPPORTED;
    // keep every plane index inside 2^31 elements per (sequence, head) and
    // the grid dimensions inside their limits
    if ((long long)c->max_tokens > (1LL << 24) || (long long)c->batch * c->q_heads > (1LL << 24) ||
        (long long)c->batch * c->kv_heads * (qpk / kvqi::block_heads(qpk)) > 65535 ||
        ((c->geometry != 0 || c->format != KVQ_FORMAT_INT) &&
         (long long)c->batch * c->q_heads > 65535))  // one block row per output row
        return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

void make_layout(const kvq_config* c, kvq_layout* L)
{
    const size_t nb = c->batch, hkv = c->kv_heads, hq = c->q_heads, D = c->head_dim;
    const size_t G = c->group;
    const int gcap = (c->max_tokens + c->group - 1) / c->group;
    const size_t tcap = (size_t)gcap * G;
    const size_t wk = G * c->key_bits / 32, wv = G * c->value_bits / 32;
    const size_t esz = c->dtype == KVQ_F16 ? 2 : 4;
    int ms = (kTargetBlocks + (int)(nb * hkv) - 1) / (int)(nb * hkv);
    if (ms > kMaxSplits) ms = kMaxSplits;
    if (ms > gcap + 1) ms = gcap + 1;
    if (ms < 1) ms = 1;
    size_t off = 0;
    L->k_codes = off;   off = align_up(off + nb * hkv * gcap * D * wk * 4);
    L->k_meta = off;    off = align_up(off + nb * hkv * gcap * D * 4);
    L->v_codes = off;   off = align_up(off + nb * hkv * tcap * (D / G) * wv * 4);
    L->v_meta = off;    off = align_up(off + nb * hkv * tcap * (D / G) * 4);
    const size_t ring = (size_t)c->residual + G;
    L->k_tail = off;    off = align_up(off + nb * hkv * ring * D * esz);
    const bool v_ring = c->residual > 0 || (c->geometry & KVQ_VALUES_PER_CHANNEL) != 0;
    L->v_tail = off;    off = align_up(off + (v_ring ? nb * hkv * ring * D * esz : 0));
    L->k_sink = off;    off = align_up(off + nb * hkv * (size_t)c->sink * D * esz);
    L->v_sink = off;    off = align_up(off + nb * hkv * (size_t)c->sink * D * esz);
    L->rope_group = off; off = align_up(off + (size_t)gcap * (D / 2) * 8);
    L->rope_offset = off; off = align_up(off + G * (D / 2) * 8);
    L->partials = off;  off = align_up(off + nb * hq * (size_t)ms * (D + 2) * 4);
    L->total_bytes = off;
    L->gcap = gcap;
    L->tcap = (int32_t)tcap;
    L->max_splits = ms;
    L->tail_slots = (int32_t)ring;
}

kvqi::Planes planes_of(const kvq* h)
{
    const kvq_layout& L = h->layout;
    kvqi::Planes p;
    p.k_codes = reinterpret_cast<uint32_t*>(h->ws + L.k_codes);
    p.k_meta = reinterpret_cast<uint32_t*>(h->ws + L.k_meta);
    p.v_codes = reinterpret_cast<uint32_t*>(h->ws + L.v_codes);
    p.v_meta = reinterpret_cast<uint32_t*>(h->ws + L.v_meta);
    p.k_tail = h->ws + L.k_tail;
    p.v_tail = h->ws + L.v_tail;
    p.k_sink = h->ws + L.k_sink;
    p.v_sink = h->ws + L.v_sink;
    p.rope_group = reinterpret_cast<const float2*>(h->ws + L.rope_group);
    p.rope_offset = reinterpret_cast<const float2*>(h->ws + L.rope_offset);
    p.partials = reinterpret_cast<float*>(h->ws + L.partials);
    p.nb = h->cfg.batch;
    p.hq = h->cfg.q_heads;
    p.hkv = h->cfg.kv_heads;
    p.D = h->cfg.head_dim;
    p.kbits = h->cfg.key_bits;
    p.vbits = h->cfg.value_bits;
    p.gcap = L.gcap;
    p.tcap = L.tcap;
    p.max_splits = L.max_splits;
    p.dtype = h->cfg.dtype;
    p.residual = h->cfg.residual;
    p.ring = L.tail_slots;
    p.sink = h->cfg.sink;
    p.geometry = h->cfg.geometry;
    p.rope_base = h->cfg.rope_base;
    p.format = h->cfg.format;
    return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

int env_int(const char* name)
{
    const char* v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

// The status of a call that enqueued work with status st: in debug-sync mode
// the stream is drained and the runtime's error state read, so a fault in
// that work is reported here.
int settle(const kvq* h, void* stream, int st)
{
    if (st != KVQ_OK || !h->sync)
        return st;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    const hipError_t last = hipGetLastError();
    if (e == hipSuccess)
        e = last;
    return hip_status(e);
}

// Launch shape of the decode-attention kernel.  A compute unit holds 16
// waves of the one-query-head kernel (8 when several query heads share a
// KV head: more registers).  Best measured: blocks of that full size, with
// splits chosen so that blocks = k * CUs for a small k (every CU gets the
// same whole number of blocks).  Without such a fit: 8-wave blocks and at
// least two splits for the variants with row-DPP sums (no LDS reduce
// buffers) when there are fewer than 4 units per CU (13B shape 147-150 us
// against 151-153 us with 4-wave blocks; larger counts were not measured);
// otherwise 4-wave blocks and enough splits for about three blocks per CU,
// which keeps the last round short (their reduce buffers limit larger
// blocks to one per CU: 211-215 us against 180-183 us at 4-bit values).
void attend_shape(const kvq* h, int n, int* splits_out, int* waves_out)
{
    const int qpk_all = h->cfg.q_heads / h->cfg.kv_heads;
    const int units = h->cfg.batch * h->cfg.kv_heads * (qpk_all / kvqi::block_heads(qpk_all));
    const int cus = h->cus > 0 ? h->cus : 256;
    // quantized groups: [sink/G, Tq/G), none while n < sink
    const int qg = kvqi::quantized_end(n, h->cfg.residual, h->cfg.sink) / h->cfg.group -
                   h->cfg.sink / h->cfg.group;
    const int full_groups = qg > 0 ? qg : 0;
    const int groups_per_step = 64 / (h->cfg.head_dim / 2);
    const int wpc = kvqi::max_block_waves(kvqi::block_heads(qpk_all));
    const int cap = full_groups > 0 ? full_groups : 1;
    const int max_splits = h->layout.max_splits < cap ? h->layout.max_splits : cap;
    int splits = 0, waves = 0;
    for (int k = 1; k <= 4 && splits == 0; ++k) {
        if ((long long)k * cus % units != 0)
            continue;
        const long long sp = (long long)k * cus / units;
        if (sp >= 1 && sp <= max_splits) {
            splits = (int)sp;
            waves = wpc;
        }
    }
    if (splits == 0) {
        // (the 8-wave rule where it was measured: fewer units than 4 per CU)
        const bool rowdpp = kvqi::row_dpp_sums(h->cfg.head_dim, h->cfg.key_bits,
                                               h->cfg.value_bits, kvqi::block_heads(qpk_all)) &&
                            units < 4 * cus;
        waves = rowdpp ? 8 : 4;
        splits = (int)(((long long)(wpc / waves) * cus + units - 1) / units);
        if (rowdpp && splits < 2)
            splits = 2;
        if (splits > max_splits)
            splits = max_splits;
        if (splits < 1)
            splits = 1;
    }
    if (h->force_splits > 0)
        splits = h->force_splits < max_splits ? h->force_splits : max_splits;
    // waves beyond the groups of a block would idle
    const int per_block = (full_groups + splits - 1) / splits;
    const int useful = (per_block + groups_per_step - 1) / groups_per_step;
    if (waves > useful)
        waves = useful;
    if (h->force_waves > 0)
        waves = h->force_waves;
    if (waves > wpc)
        waves = wpc;
    if (waves < 1)
        waves = 1;
    *splits_out = splits;
    *waves_out = waves;
}

// Decode attention over the geometry-ablation and FP8 caches: about
// kTargetBlocks blocks, at least one 32-token chunk per split.
bool other_path(const kvq* h)
{
    return h->cfg.geometry != 0 || h->cfg.format != KVQ_FORMAT_INT;
}

// Splits and waves of the decode attention at length n; `fused`: the launch
// also appends token n-1 (threads 0 .. head_dim-1 of the last split).
void plan_attend(const kvq* h, int n, bool fused, int* splits_out, int* waves_out)
{
    if (other_path(h)) {
        const int rows = h->cfg.batch * h->cfg.q_heads;
        const int chunks = (n + h->cfg.group - 1) / h->cfg.group;
        int splits = (kTargetBlocks + rows - 1) / rows;
        if (h->force_splits > 0) splits = h->force_splits;
        if (splits > chunks) splits = chunks;
        if (splits > h->layout.max_splits) splits = h->layout.max_splits;
        if (splits < 1) splits = 1;
        *splits_out = splits;
        *waves_out = 0;
        return;
    }
    attend_shape(h, n, splits_out, waves_out);
    const int append_waves = h->cfg.head_dim / 64;
    if (fused && *waves_out < append_waves)
        *waves_out = append_waves;
}

// Bytes of split partials a launch with `splits` splits writes (none with
// one split: it writes the output itself).
size_t partial_bytes(const kvq* h, int splits)
{
    return splits > 1 ? (size_t)h->cfg.batch * h->cfg.q_heads * splits *
                            (h->cfg.head_dim + 2) * sizeof(float)
                      : 0;
}

// Enqueue the decode attention at length n (with k_new/v_new: the fused
// append of token n-1).  The split partials go to the workspace's region,
// or with use_static to the library's static scratch, packed with a stride
// of `splits` per output row.
int launch_attend(kvq* h, int n, int splits, int waves, const void* q, float* out,
                  const void* k_new, const void* v_new, hipStream_t s, bool use_static)
{
    kvqi::Planes p = planes_of(h);
    if (use_static) {
        p.partials = h->scratch;
        p.max_splits = splits;
    }
    if (other_path(h))
        return hip_status(h->cfg.format == KVQ_FORMAT_FP8_E4M3
                              ? kvqi::launch_attend_fp8(p, q, out, n, splits, s)
                              : kvqi::launch_attend_geometry(p, q, out, n, splits, s));
    return hip_status(h->cfg.head_dim == 64
                          ? kvqi::launch_attend_d64(p, q, out, n, splits, waves, k_new, v_new, s)
                          : kvqi::launch_attend_d128(p, q, out, n, splits, waves, k_new, v_new,
                                                     s));
}

// One decode step: append, then attend.  One launch for a plain cache with
// at most 4 query heads per KV head (one block per KV head), else the two
// calls.  Everything is checked before anything is enqueued.
int append_attend(kvq* h, const void* d_k, const void* d_v, const void* d_q, float* d_out,
                  void* stream, bool use_static)
{
    if (!h || !d_k || !d_v || !d_q || !d_out)
        return KVQ_ERR_ARG;
    if (h->n >= h->cfg.max_tokens)
        return KVQ_ERR_CAPACITY;
    const int qpk_all = h->cfg.q_heads / h->cfg.kv_heads;
    const bool fused = h->cfg.residual == 0 && h->cfg.sink == 0 && h->cfg.geometry == 0 &&
                       h->cfg.format == KVQ_FORMAT_INT &&
                       kvqi::block_heads(qpk_all) == qpk_all;  // one block per KV head
    const int n = h->n + 1;
    int splits, waves;
    plan_attend(h, n, fused, &splits, &waves);
    if (use_static && (!h->scratch || partial_bytes(h, splits) > kvqi::kStaticScratchBytes))
        return h->scratch ? KVQ_ERR_SCRATCH : KVQ_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!fused) {
        const int st = kvq_append_token(h, d_k, d_v, stream);
        return st != KVQ_OK ? st
                            : settle(h, stream,
                                     launch_attend(h, n, splits, waves, d_q, d_out, nullptr,
                                                   nullptr, s, use_static));
    }
    const int st =
        settle(h, stream, launch_attend(h, n, splits, waves, d_q, d_out, d_k, d_v, s, use_static));
    if (st == KVQ_OK)
        h->n = n;
    return st;
}

}  // namespace

extern "C" {

size_t kvq_workspace_bytes(const kvq_config* cfg)
{
    if (check_config(cfg) != KVQ_OK)
        return 0;
    kvq_layout L;
    make_layout(cfg, &L);
    return L.total_bytes;
}

int kvq_layout_for(const kvq_config* cfg, kvq_layout* out)
{
    if (!out)
        return KVQ_ERR_ARG;
    const int st = check_config(cfg);
    if (st != KVQ_OK)
        return st;
    make_layout(cfg, out);
    return KVQ_OK;
}

int kvq_create(const kvq_config* cfg, void* d_ws, size_t ws_bytes, kvq_t** out)
{
    if (!out || !d_ws)
        return KVQ_ERR_ARG;
    const int st = check_config(cfg);
    if (st != KVQ_OK)
        return st;
    kvq_layout L;
    make_layout(cfg, &L);
    if (ws_bytes < L.total_bytes || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) != 0)
        return KVQ_ERR_WORKSPACE;
    // Rotary tables, computed in fp64 and stored as fp32 (cos, sin):
    //   group table  [g][i] = angle g*G*theta_i,  offset table [j][i] = j*theta_i,
    // theta_i = base^(-2i/D); position p = g*G + j composes as a product.
    const int D = cfg->head_dim, NP = D / 2, G = cfg->group;
    std::vector<float> grp((size_t)L.gcap * NP * 2), offs((size_t)G * NP * 2);
    for (int i = 0; i < NP; ++i) {
        const double theta = std::pow((double)cfg->rope_base, -2.0 * i / (double)D);
        for (int g = 0; g < L.gcap; ++g) {
            const double a = (double)g * G * theta;
            grp[((size_t)g * NP + i) * 2] = (float)std::cos(a);
            grp[((size_t)g * NP + i) * 2 + 1] = (float)std::sin(a);
        }
        for (int j = 0; j < G; ++j) {
            const double a = (double)j * theta;
            offs[((size_t)j * NP + i) * 2] = (float)std::cos(a);
            offs[((size_t)j * NP + i) * 2 + 1] = (float)std::sin(a);
        }
    }
    char* ws = static_cast<char*>(d_ws);
    if (hipMemcpy(ws + L.rope_group, grp.data(), grp.size() * sizeof(float),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ws + L.rope_offset, offs.data(), offs.size() * sizeof(float),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        return KVQ_ERR_HIP;
    // the static scratch's address on this device, looked up once per device
    int dev = 0;
    void* scratch = nullptr;
    if (hipGetDevice(&dev) != hipSuccess || kvqi::static_scratch(dev, &scratch) != hipSuccess)
        return KVQ_ERR_HIP;
    kvq* h = new (std::nothrow) kvq;
    if (!h)
        return KVQ_ERR_ARG;
    h->cfg = *cfg;
    h->layout = L;
    h->ws = ws;
    h->n = 0;
    h->cus = 0;
    h->scratch = static_cast<float*>(scratch);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
        h->cus = prop.multiProcessorCount;
    h->force_splits = env_int("KVQ_ATTEND_SPLITS");
    h->force_waves = env_int("KVQ_ATTEND_WAVES");
    h->sync = env_int("KVQ_SYNC") == 1;
    *out = h;
    return KVQ_OK;
}

int kvq_quantize_prefill(kvq_t* h, const void* d_k, const void* d_v, int32_t n_tokens,
                         void* stream)
{
    if (!h || n_tokens < 0)
        return KVQ_ERR_ARG;
    if (n_tokens > 0 && (!d_k || !d_v))
        return KVQ_ERR_ARG;
    if (h->n != 0)
        return KVQ_ERR_STATE;
    if (n_tokens > h->cfg.max_tokens)
        return KVQ_ERR_CAPACITY;
    if (n_tokens == 0)
        return KVQ_OK;
    const kvqi::Planes p = planes_of(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int st = settle(h, stream,
                          hip_status(p.format == kvqi::kFormatFp8
                                         ? kvqi::launch_fp8_prefill(p, d_k, d_v, n_tokens, s)
                                         : kvqi::launch_quantize_prefill(p, d_k, d_v, n_tokens, s)));
    if (st == KVQ_OK)
        h->n = n_tokens;
    return st;
}

int kvq_append_token(kvq_t* h, const void* d_k, const void* d_v, void* stream)
{
    if (!h || !d_k || !d_v)
        return KVQ_ERR_ARG;
    if (h->n >= h->cfg.max_tokens)
        return KVQ_ERR_CAPACITY;
    const kvqi::Planes p = planes_of(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int st = settle(h, stream,
                          hip_status(p.format == kvqi::kFormatFp8
                                         ? kvqi::launch_fp8_append(p, d_k, d_v, h->n, s)
                                         : kvqi::launch_append(p, d_k, d_v, h->n, s)));
    if (st == KVQ_OK)
        h->n += 1;
    return st;
}

int kvq_attend_decode(kvq_t* h, const void* d_q, float* d_out, void* stream)
{
    if (!h || !d_q || !d_out)
        return KVQ_ERR_ARG;
    if (h->n == 0)
        return KVQ_ERR_STATE;
    int splits, waves;
    plan_attend(h, h->n, false, &splits, &waves);
    return settle(h, stream,
                  launch_attend(h, h->n, splits, waves, d_q, d_out, nullptr, nullptr,
                                static_cast<hipStream_t>(stream), false));
}

int kvq_append_attend(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                      float* d_out, void* stream)
{
    return append_attend(h, d_k, d_v, d_q, d_out, stream, false);
}

int kvq_append_attend_static(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                             float* d_out, void* stream)
{
    return append_attend(h, d_k, d_v, d_q, d_out, stream, true);
}

int kvq_error_metrics(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                      double* d_metrics, void* stream)
{
    if (!h || !d_k || !d_v || !d_q || !d_metrics)
        return KVQ_ERR_ARG;
    if (h->n == 0)
        return KVQ_ERR_STATE;
    if (h->cfg.format != KVQ_FORMAT_INT)
        return KVQ_ERR_UNSUPPORTED;
    return settle(h, stream,
                  hip_status(kvqi::launch_error_metrics(planes_of(h), d_k, d_v, d_q, d_metrics,
                                                        h->n, static_cast<hipStream_t>(stream))));
}

int kvq_destroy(kvq_t* h)
{
    if (!h)
        return KVQ_ERR_ARG;
    delete h;
    return KVQ_OK;
}

int32_t kvq_length(const kvq_t* h) { return h ? h->n : -1; }

int kvq_get_layout(const kvq_t* h, kvq_layout* out)
{
    if (!h || !out)
        return KVQ_ERR_ARG;
    *out = h->layout;
    return KVQ_OK;
}

const char* kvq_strerror(int status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case KVQ_ERR_STATE: return "call not valid in the cache's current state";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_SCRATCH: return "the call needs more than the library's static device scratch";
    default: return "unknown status";
    }
}

}  // extern "C"
