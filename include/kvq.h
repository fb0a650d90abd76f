/*
 * kvq.h -- C ABI of the MI355X (gfx950) library for a KIVI-style asymmetric
 * quantized KV cache and the decode attention that reads it.
 *
 * The method (from the web pages this library implements):
 *   - uniform asymmetric integer quantization of a group: zero point = the
 *     group's minimum, step = range / (2^B - 1), every element rounded to the
 *     nearest step ("Your KV Cache Doesn't Have a Bit Problem. It Has a
 *     Geometry Problem", section "What Quantization Error Is Actually Made
 *     Of");
 *   - keys grouped per channel over runs of G consecutive tokens, values per
 *     token over runs of G consecutive channels (same page, sections "Keys:
 *     The Outliers Live in Fixed Channels" and "Values: Where the Intuition
 *     Breaks"; "Why KV Cache Geometry Matters More Than Bit Precision for
 *     LLM Speed", section "Stop Obsessing Over Bits");
 *   - key tokens that do not yet fill a group wait unquantized in a tail
 *     buffer and are quantized as a group once G have accumulated; values
 *     are quantized as each token arrives ("...Bit Problem...", section "The
 *     Systems Tax, and Why It Is Not a Detail");
 *   - keys are quantized before the rotary position embedding, which is
 *     applied after dequantization inside attention ("...Bit Problem...",
 *     section "Rotary Embeddings Complicate the Keys");
 *   - decode attention reads the whole cache for every generated token
 *     ("...Bit Problem...", section "Why the KV Cache Is Where This Bites").
 *
 * Conventions shared by every entry point
 *   - All pointers named d_* are device (HIP) pointers; everything else is
 *     host memory.  The caller owns every buffer, including the workspace;
 *     the library never allocates or frees device memory.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call except kvq_create only enqueues work on that stream and returns;
 *     results are valid once the caller has synchronized it.  Calls on one
 *     handle must be ordered on one stream by the caller.  A handle is not
 *     thread-safe.
 *   - Every function returns KVQ_OK (0) or a negative KVQ_ERR_* code.  All
 *     argument and state checks run before anything is enqueued: on error the
 *     handle's state is unchanged and no GPU work was queued.
 *   - Debugging: with the environment variable KVQ_SYNC set to 1 when a
 *     handle is created, every call on that handle that enqueues work then
 *     synchronizes its stream and checks the runtime's error state, so a
 *     kernel fault is reported (KVQ_ERR_HIP, handle state not advanced) by
 *     the call that caused it.  Not for use under stream capture.
 *   - Element types (kvq_config.dtype): KVQ_F16 (IEEE binary16) or KVQ_F32.
 *     Keys, values, queries and the key tail use that type; the output is
 *     always fp32.  Non-finite inputs are undefined behaviour.
 *   - Supported: group == 32; key_bits, value_bits in {2, 4, 8};
 *     head_dim in {64, 128}; q_heads a multiple of kv_heads with
 *     q_heads / kv_heads in {1, 2, 4, 8}.
 *
 * Packed planes inside the workspace (byte offsets from kvq_get_layout; each
 * plane 256-byte aligned).  Gcap = ceil(max_tokens / G), Tcap = Gcap * G,
 * Wk = G * key_bits / 32, Wv = G * value_bits / 32 (32-bit words per group):
 *   K_CODES u32[batch][kv_heads][Gcap][head_dim][Wk]
 *           code of token j of key group g, channel c, at bits
 *           [j*key_bits, j*key_bits + key_bits) of the Wk-word little-endian
 *           bit string (word j*key_bits/32, LSB first)
 *   K_META  u32[batch][kv_heads][Gcap][head_dim]
 *           binary16 step in bits 0..15, binary16 zero point in bits 16..31
 *   V_CODES u32[batch][kv_heads][Tcap][head_dim/G][Wv]
 *           code of channel cg*G + j of token t at bits [j*value_bits, ...)
 *   V_META  u32[batch][kv_heads][Tcap][head_dim/G]   (as K_META)
 *   K_TAIL  dtype[batch][kv_heads][R+G][head_dim]
 *           ring: key token t >= Tq verbatim in slot t mod (R+G)
 *   V_TAIL  dtype[batch][kv_heads][R+G][head_dim]   (R > 0 only, else empty)
 *           ring: value token t >= Tq verbatim in slot t mod (R+G)
 *   K_SINK  dtype[batch][kv_heads][S][head_dim]     (S = kvq_config.sink)
 *   V_SINK  dtype[batch][kv_heads][S][head_dim]
 *           key / value token t < min(n, S) verbatim in slot t
 * Residual window R = kvq_config.residual (the page "Your KV Cache Doesn't
 * Have a Bit Problem...", section "The Systems Tax, and Why It Is Not a
 * Detail": KIVI keeps the most recent tokens in full precision).  Tokens
 * [0, Tq) are quantized, Tq = G * floor(max(0, n - R) / G); tokens [Tq, n)
 * stay in full precision: their keys always, their values when R > 0 (with
 * R = 0 every value is quantized on arrival and only the < G keys of the
 * unfilled group wait).  With R > 0 at least R and at most R + G - 1 recent
 * tokens are unquantized; a G-block is quantized when it leaves the window.
 * Sink window S = kvq_config.sink (same page, section "Where the Work Is
 * Headed": InnerQ keeps high-precision windows for the recent tokens and the
 * attention-sink tokens): keys and values of tokens [0, min(n, S))
 * stay unquantized for good, quantization starts at token S, and Tq above is
 * raised to at least min(n, S).
 * Geometry ablation, kvq_config.geometry (the page "Your KV Cache Doesn't Have
 * a Bit Problem...", lede and sections "Keys: The Outliers Live in Fixed
 * Channels" and "Values: Where the Intuition Breaks": the same bits spent
 * along the other axis).  0 is the layout above.  KVQ_KEYS_PER_TOKEN groups
 * keys like values (G channels of one token, quantized on arrival): K_CODES
 * is u32[batch][kv_heads][Tcap][head_dim/G][Wk] and K_META
 * u32[batch][kv_heads][Tcap][head_dim/G], and the key tail is unused.
 * KVQ_VALUES_PER_CHANNEL groups values like keys (one channel over G
 * tokens): V_CODES is u32[batch][kv_heads][Gcap][head_dim][Wv], V_META
 * u32[batch][kv_heads][Gcap][head_dim], and value tokens t >= G*floor(n/G)
 * wait verbatim in V_TAIL (G slots, token t in slot t mod G) until their
 * group fills.  Plane sizes do not change.  A non-zero geometry requires
 * residual == sink == 0; its attention runs in a separate, plain kernel.
 * FP8 cache, kvq_config.format == KVQ_FORMAT_FP8_E4M3 (the page "Rotate,
 * Then Round: The Geometry of KV-Cache Compression", key takeaways: FP8 as
 * the production default): every key and value element is one OCP FP8 E4M3
 * byte (bias 7, largest finite 448, no infinities), rounded to nearest with
 * ties to even and saturated at +-448, no scale factor; keys before the
 * rotary embedding.  K_CODES and V_CODES (sized for 8-bit codes) hold one
 * head_dim * 32-byte block per (sequence, KV head, 32-token group g),
 * u8[batch][kv_heads][Gcap][head_dim * 32], in 16-byte pieces: channel c of
 * token gG + j at byte ((2 (c % 2) + j / 16) (head_dim / 2) + c / 2) * 16
 * + j % 16 of the block; bytes of the last group past n are 0; K_META,
 * V_META and the tails are unused.  Its
 * attention runs in a separate kernel; kvq_error_metrics does not take it.
 * The step and zero are each rounded once, to nearest-even, from the exact
 * value (range/(2^B-1) and the minimum); the code of x is the integer nearest
 * to (x - zero)/step computed exactly, ties to even, clamped to
 * [0, 2^B - 1]; a zero step gives code 0.
 *
 * Rotary embedding: channels (2i, 2i+1) form a pair rotated by the angle
 * p * rope_base^(-2i/head_dim); key token t at position t, the query at
 * position n-1 (n = cached tokens, the newest token included).  Scores are
 * scaled by 1/sqrt(head_dim); query head h reads KV head
 * h / (q_heads / kv_heads).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVQ_OK = 0,
    KVQ_ERR_ARG = -1,         /* null pointer, bad dimension, bad value     */
    KVQ_ERR_UNSUPPORTED = -2, /* valid but not built: bits, G, head_dim ... */
    KVQ_ERR_WORKSPACE = -3,   /* workspace too small or not 256-B aligned   */
    KVQ_ERR_STATE = -4,       /* prefill on a non-empty cache, attend on an
                                 empty one                                  */
    KVQ_ERR_CAPACITY = -5,    /* the call would exceed max_tokens           */
    KVQ_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    KVQ_ERR_SCRATCH = -7      /* the call needs more than the library's
                                 static device scratch (KVQ_STATIC_SCRATCH_BYTES) */
};

/* Bytes of the library's static device scratch (kvq_append_attend_static). */
#define KVQ_STATIC_SCRATCH_BYTES (4u << 20)

enum { KVQ_F16 = 0, KVQ_F32 = 1 };

/* kvq_config.format: integer codes (the method above) or FP8 E4M3 bytes. */
enum { KVQ_FORMAT_INT = 0, KVQ_FORMAT_FP8_E4M3 = 1 };

/* kvq_config.geometry bits (0 = keys per channel, values per token). */
enum { KVQ_KEYS_PER_TOKEN = 1, KVQ_VALUES_PER_CHANNEL = 2 };

/* Entries of the kvq_error_metrics result. */
enum {
    KVQ_METRIC_KEY_ERROR = 0,
    KVQ_METRIC_SCORE_ERROR = 1,
    KVQ_METRIC_VALUE_ERROR = 2,
    KVQ_METRIC_VALUE_OUTPUT_REL_ERROR = 3,
    KVQ_METRIC_OUTPUT_REL_ERROR = 4,
    KVQ_METRICS = 5
};

typedef struct kvq_config {
    int32_t batch;      /* sequences, >= 1                                  */
    int32_t q_heads;    /* query heads, multiple of kv_heads                */
    int32_t kv_heads;   /* key/value heads, >= 1                            */
    int32_t head_dim;   /* D: 64 or 128                                     */
    int32_t max_tokens; /* per-sequence capacity, >= 1                      */
    int32_t group;      /* G: must be 32                                    */
    int32_t key_bits;   /* 2, 4 or 8                                        */
    int32_t value_bits; /* 2, 4 or 8                                        */
    int32_t dtype;      /* KVQ_F16 or KVQ_F32                               */
    float rope_base;    /* > 1, e.g. 10000                                  */
    int32_t residual;   /* R: recent tokens kept in full precision, a
                           multiple of group in [0, 1024]; 0 = none         */
    int32_t sink;       /* S: first tokens kept in full precision, a
                           multiple of group in [0, 1024]; 0 = none         */
    int32_t geometry;   /* 0, or KVQ_KEYS_PER_TOKEN | KVQ_VALUES_PER_CHANNEL
                           (ablation; needs residual == sink == 0)          */
    int32_t format;     /* KVQ_FORMAT_INT (0) or KVQ_FORMAT_FP8_E4M3 (needs
                           key_bits == value_bits == 8, no windows,
                           geometry 0)                                      */
} kvq_config;

typedef struct kvq_layout {
    size_t k_codes, k_meta, v_codes, v_meta, k_tail, v_tail; /* byte offsets */
    size_t k_sink, v_sink;
    size_t rope_group, rope_offset, partials;
    size_t total_bytes;   /* == kvq_workspace_bytes(cfg)                     */
    int32_t gcap, tcap;   /* Gcap and Tcap above                             */
    int32_t max_splits;   /* token splits per (sequence, KV head) at most    */
    int32_t tail_slots;   /* R + G: slots of each tail ring                  */
} kvq_layout;

typedef struct kvq kvq_t; /* opaque; lives in host memory */

/* Bytes of device workspace a cache with this configuration needs (pure
 * host; 0 if the configuration is invalid or unsupported). */
size_t kvq_workspace_bytes(const kvq_config* cfg);

/* Create a cache handle over a caller-owned device workspace d_ws of
 * ws_bytes bytes (>= kvq_workspace_bytes, 256-byte aligned).  Writes the
 * rotary tables into the workspace with a blocking copy on the null stream
 * (the only blocking call) and sets the cached length n to 0.  The
 * workspace contents are otherwise not initialised.  *out receives the
 * handle (host memory, freed by kvq_destroy).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP. */
int kvq_create(const kvq_config* cfg, void* d_ws, size_t ws_bytes,
               kvq_t** out);

/* Quantize a whole prompt of n_tokens tokens into the empty cache.
 * d_k, d_v: dtype[batch][kv_heads][n_tokens][head_dim], keys before the
 * rotary embedding.  With Tq as above for n = n_tokens: tokens
 * t < min(n, S) go to the sinks; key groups S/G <= g < Tq/G are quantized
 * per channel (K_CODES, K_META) and keys t >= Tq go to the K_TAIL ring;
 * R = 0: every value token t >= S is quantized per channel group (V_CODES,
 * V_META); R > 0: values S <= t < Tq are quantized and values t >= Tq go to
 * the V_TAIL ring.  A non-zero geometry quantizes every token of an operand
 * grouped per token, and the groups g < n_tokens/G of one grouped per
 * channel (the rest to its tail).  Sets n = n_tokens.
 * n_tokens == 0 is allowed and enqueues nothing.
 * Errors: KVQ_ERR_ARG (null handle or pointers with n_tokens > 0, negative
 * n_tokens), KVQ_ERR_STATE (n != 0), KVQ_ERR_CAPACITY (n_tokens >
 * max_tokens), KVQ_ERR_HIP. */
int kvq_quantize_prefill(kvq_t* h, const void* d_k, const void* d_v,
                         int32_t n_tokens, void* stream);

/* Append one token per sequence: d_k, d_v are dtype[batch][kv_heads]
 * [head_dim].  With a non-zero geometry, an operand grouped per token is
 * quantized at once and one grouped per channel goes to tail slot n mod G,
 * its group quantized when n+1 is a multiple of G.  Otherwise:
 * while n < S key and value go to sink slot n.  Otherwise,
 * R = 0: the value is quantized at once; the key goes to tail
 * slot n mod G, and when that fills the tail (n+1 a multiple of G) the G
 * tail keys are quantized as key group n/G in the same launch.  R > 0: key
 * and value go to ring slot n mod (R+G); when n+1-R reaches a positive
 * multiple of G, the G-block b = (n+1-R)/G - 1 leaves the window and its
 * keys (group b) and values (tokens bG .. bG+G-1) are quantized from the
 * rings in the same launch (a block inside the sink, bG < S, is not).  Sets
 * n = n + 1.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_CAPACITY (n == max_tokens), KVQ_ERR_HIP. */
int kvq_append_token(kvq_t* h, const void* d_k, const void* d_v,
                     void* stream);

/* Decode attention of one query per head over all n cached tokens.
 * d_q: dtype[batch][q_heads][head_dim], before the rotary embedding.
 * d_out: float[batch][q_heads][head_dim].  Uses the workspace's partials
 * region as scratch, so two attend calls on one handle must not run
 * concurrently.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE (n == 0), KVQ_ERR_HIP. */
int kvq_attend_decode(kvq_t* h, const void* d_q, float* d_out, void* stream);

/* One decode step: kvq_append_token(h, d_k, d_v) followed by
 * kvq_attend_decode(h, d_q, d_out) over the n + 1 tokens, with the same
 * arguments, layouts, results and state change (n = n + 1).  The pages
 * describe exactly this order per generated token: the new key and value
 * join the cache, then attention reads all of it ("Your KV Cache Doesn't
 * Have a Bit Problem...", sections "Why the KV Cache Is Where This Bites"
 * and "The Systems Tax, and Why It Is Not a Detail").  For a cache without
 * windows (residual == sink == 0), geometry 0, integer codes and at most 4
 * query heads per KV head, both run in one kernel launch: the block that
 * reads the newest tokens appends them first.  Otherwise the two calls are
 * made in turn.  Results equal those of the two calls up to the order of
 * fp32 additions (the launch may use more waves).
 * Errors: KVQ_ERR_ARG (a null pointer), KVQ_ERR_CAPACITY (n == max_tokens),
 * KVQ_ERR_HIP; validation precedes any enqueue.  In the two-call form a
 * KVQ_ERR_HIP from the attention leaves the append done (n = n + 1). */
int kvq_append_attend(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                      float* d_out, void* stream);

/* kvq_append_attend for callers that cannot allocate device memory or touch
 * the workspace's scratch region while the call runs (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step with the same arguments, kernels, launch shape, results and state
 * change, except that the decode attention's split partials live in the
 * library's own static device array of KVQ_STATIC_SCRATCH_BYTES (4 MiB) per
 * GPU instead of the workspace's partials region.  The call allocates
 * nothing.  A step that splits the token range S > 1 ways needs
 * batch * q_heads * S * (head_dim + 2) * 4 bytes of it; one that does not
 * split needs none.  The array is found at kvq_create (once per device, with
 * that device current) and kept until the process ends; it keeps the last
 * call's contents, and every call on one GPU shares it, so calls that
 * overlap on one GPU (several streams, several threads) race.
 * Errors: as kvq_append_attend, and KVQ_ERR_SCRATCH when the step would need
 * more than the array holds (nothing enqueued, n unchanged). */
int kvq_append_attend_static(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                             float* d_out, void* stream);

/* Error where it is consumed (the page "Your KV Cache Doesn't Have a Bit
 * Problem...", sections "Keys: The Outliers Live in Fixed Channels" and
 * "Values: Where the Intuition Breaks": validate on attention, not on the
 * stored tensor), computed in fp64 for the current cache of n tokens.
 * d_k, d_v: dtype[batch][kv_heads][n][head_dim], the unquantized keys
 * (before the rotary embedding) and values of all n cached tokens, i.e.
 * what prefill and the appends received, in order.  d_q: as for
 * kvq_attend_decode.  d_metrics: double[KVQ_METRICS], each entry a mean over
 * the batch * q_heads output rows; with a = softmax of the scores from the
 * unquantized keys, ahat the same from the stored keys (dequantized codes,
 * or the verbatim tail, ring and sink rows), vhat the stored values:
 *   KEY_ERROR               Frobenius norm of khat - k over the row's KV head
 *                           (before the rotation);
 *   SCORE_ERROR             L2 norm of ahat - a;
 *   VALUE_ERROR             Frobenius norm of vhat - v over the row's KV head;
 *   VALUE_OUTPUT_REL_ERROR  |sum_t a_t vhat_t - sum_t a_t v_t| / |sum_t a_t v_t|;
 *   OUTPUT_REL_ERROR        |sum_t ahat_t vhat_t - sum_t a_t v_t| / |sum_t a_t v_t|.
 * Uses the workspace's partials region as scratch (like kvq_attend_decode:
 * not concurrently with another attend or metrics call on the handle).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_STATE (n == 0), KVQ_ERR_UNSUPPORTED (an FP8
 * cache), KVQ_ERR_HIP. */
int kvq_error_metrics(kvq_t* h, const void* d_k, const void* d_v, const void* d_q,
                      double* d_metrics, void* stream);

/* Free the handle (host memory only; the workspace is untouched).
 * Errors: KVQ_ERR_ARG (null). */
int kvq_destroy(kvq_t* h);

/* Cached tokens n (pure host; -1 for a null handle). */
int32_t kvq_length(const kvq_t* h);

/* Plane offsets inside the workspace (pure host).  Errors: KVQ_ERR_ARG. */
int kvq_get_layout(const kvq_t* h, kvq_layout* out);

/* Workspace layout for a configuration without a handle (pure host).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED. */
int kvq_layout_for(const kvq_config* cfg, kvq_layout* out);

/* Static description of a status code (pure host). */
const char* kvq_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
