// kvq_internal.h -- declarations shared by the host API (kvq_host.cpp) and
// the gfx950 kernels (kvq_kernels.hip).  Not part of the public ABI.
#pragma once

#include "kvq.h"

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvqi {

constexpr int kGroup = 32;  // G: tokens per key group, channels per value group

// Largest attention block in waves: 16 (up to 128 VGPRs per lane) with one
// query head per KV head, 8 (up to 256) when several query heads share one.
constexpr int max_block_waves(int qpk) { return qpk == 1 ? 16 : 8; }

// Query heads per attention block: at most 4; 8 query heads per KV head run
// as two blocks of 4 over the same KV head.
constexpr int block_heads(int qpk) { return qpk < 4 ? qpk : 4; }

// Attention variants whose per-pair partial scores are summed by DPP row
// rotations instead of through LDS (one query head per block, head_dim 128,
// 2-bit keys or 4-bit keys with 2-bit values): they need no LDS reduce
// buffers.
constexpr bool row_dpp_sums(int head_dim, int kbits, int vbits, int block_qpk)
{
    return block_qpk == 1 && head_dim == 128 && (kbits == 2 || (kbits == 4 && vbits == 2));
}

// Everything a kernel needs to address the planes of one cache.
struct Planes {
    uint32_t* k_codes;   // [nb][hkv][gcap][D][wk]
    uint32_t* k_meta;    // [nb][hkv][gcap][D]
    uint32_t* v_codes;   // [nb][hkv][tcap][D/G][wv]
    uint32_t* v_meta;    // [nb][hkv][tcap][D/G]
    void* k_tail;        // dtype[nb][hkv][ring][D]: key t >= Tq in slot t mod ring
    void* v_tail;        // dtype[nb][hkv][ring][D]: the same for values (residual > 0)
    void* k_sink;        // dtype[nb][hkv][sink][D]: key t < min(n, sink) in slot t
    void* v_sink;        // dtype[nb][hkv][sink][D]: the same for values
    const float2* rope_group;   // [gcap][D/2]  (cos, sin) of g*G*theta_i
    const float2* rope_offset;  // [G][D/2]     (cos, sin) of j*theta_i
    float* partials;     // [nb*hq][max_splits][D+2]
    int nb, hq, hkv, D, kbits, vbits, gcap, tcap, max_splits, dtype;
    int residual, ring;  // R and R + G
    int sink;            // S
    int geometry;        // 0, or kKeysPerToken | kValuesPerChannel (then R = S = 0)
    double rope_base;    // theta_i = rope_base^(-2i/D) (fp64 paths recompute angles)
    int format;          // 0: integer codes; kFormatFp8: E4M3 bytes in k_codes/v_codes
};

// FP8 (E4M3) cache: one byte per element inside the k_codes and v_codes
// planes, a D*32-byte block per (sequence, head, 32-token group) made of
// 16-byte pieces: channel c of token j at byte
// ((2*(c%2) + j/16) * D/2 + c/2) * 16 + j%16 of its block (fp8_offset).
constexpr int kFormatFp8 = 1;

// Geometry ablation bits: keys grouped like values (G channels of one token,
// planes [tcap][D/G][wk]) and values grouped like keys (one channel over G
// tokens, planes [gcap][D][wv], unfilled groups in v_tail).
constexpr int kKeysPerToken = 1;
constexpr int kValuesPerChannel = 2;

// Tq: tokens [0, Tq) of an n-token cache are quantized (keys in whole
// groups); the keys of [Tq, n), and with a residual window its values, are
// held verbatim in the tail rings.
__host__ __device__ inline int quantized_tokens(int n, int residual)
{
    const int a = n - residual;
    return a > 0 ? a / kGroup * kGroup : 0;
}

// With a sink window of S tokens: tokens [0, min(n, S)) stay in the sinks,
// [S, Tq) are quantized, [Tq, n) are in the rings; Tq >= min(n, S).
__host__ __device__ inline int quantized_end(int n, int residual, int sink)
{
    const int s = n < sink ? n : sink;
    const int q = quantized_tokens(n, residual);
    return q > s ? q : s;
}

// Bytes of the library's static device scratch (kvq_scratch.hip), which
// holds the split partials of kvq_append_attend_static.
constexpr size_t kStaticScratchBytes = KVQ_STATIC_SCRATCH_BYTES;

// Device address of that scratch on `device`, which must be current; looked
// up once per device and kept.
hipError_t static_scratch(int device, void** out);

// Launch wrappers (kvq_kernels.hip).  All enqueue on `stream` and return the
// hipGetLastError() status of the launches.
hipError_t launch_quantize_prefill(const Planes& p, const void* k, const void* v,
                                   int n_tokens, hipStream_t stream);
hipError_t launch_append(const Planes& p, const void* k, const void* v, int n,
                         hipStream_t stream);
// Decode attention over n tokens (kvq_attend_d64.hip, kvq_attend_d128.hip).
// With k_new and v_new non-null (plain cache: no windows, geometry 0,
// integer codes; one block per (sequence, KV head) and split), the kernel
// first appends token n-1 from them, as launch_append with n-1 would.
hipError_t launch_attend_d64(const Planes& p, const void* q, float* out, int n,
                             int splits, int waves, const void* k_new, const void* v_new,
                             hipStream_t stream);
hipError_t launch_attend_d128(const Planes& p, const void* q, float* out, int n,
                              int splits, int waves, const void* k_new, const void* v_new,
                              hipStream_t stream);
// Attention over a cache with a non-zero geometry (kvq_geometry.hip).
hipError_t launch_attend_geometry(const Planes& p, const void* q, float* out, int n,
                                  int splits, hipStream_t stream);
// FP8 cache (kvq_fp8.hip).
hipError_t launch_fp8_prefill(const Planes& p, const void* k, const void* v, int n,
                              hipStream_t stream);
hipError_t launch_fp8_append(const Planes& p, const void* k, const void* v, int n,
                             hipStream_t stream);
hipError_t launch_attend_fp8(const Planes& p, const void* q, float* out, int n, int splits,
                             hipStream_t stream);
// Error where it is consumed: fp64, any geometry and windows; uses the
// partials region as scratch for per-row sums (kvq_geometry.hip).
hipError_t launch_error_metrics(const Planes& p, const void* k, const void* v, const void* q,
                                double* metrics, int n, hipStream_t stream);

}  // namespace kvqi
