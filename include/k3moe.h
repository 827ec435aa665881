/*
 * k3moe — sigmoid-routed MXFP4 expert layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only. Every tensor pointer is a DEVICE
 * pointer owned by the caller; every call is asynchronous on the caller's HIP
 * stream (passed as void*, a hipStream_t; NULL is the null stream) unless its
 * comment says it synchronises.
 *
 * What the layer computes is stated on the "kimi-k3-in-c" README
 * (FareedKhan-dev): §9 "Picking 16 experts of 896" gives the router
 * (k3_router) and the layer (k3_moe, k3_situ_glu); §4 "Reduction one: the
 * experts already ship at half a byte" gives the MXFP4 weight format; §5
 * "Kernels with a floating point contract" gives k3_rmsnorm. A layer is flat
 * (latent = 0: the experts take the hidden vector directly) or latent (the
 * pages' k3_moe: the experts run in a narrow latent between a bf16 down- and
 * up-projection, with an RMSNorm on their aggregate).
 *
 * Per token x (bf16, hidden H):
 *   route:   logit[e] = Wr[e] . x                (exact products, fp64 sum;
 *                                                 T > 4: fp32 sums of runs of
 *                                                 32 products, added in fp64)
 *            sc[e] = fp32(sigmoid(fp32(logit[e])))   unbiased score
 *            ch[e] = sc[e] + bias[e]  (fp32)          selection score
 *            idx[0..k) = the k largest ch, largest first, equal ch -> lower e
 *            w[j] = sc[idx[j]]; if renorm and s = sum_j w[j] > 0: w[j] /= s;
 *            w[j] *= routed_scale                     (fp32, j order)
 *   forward (flat):
 *            out = sum_j w[j] * W2_e( act(W1_e x, W3_e x) ),  e = idx[j],
 *                  summed in router order j = 0..k-1, then
 *            out += S2( act(S1 x, S3 x) )             shared expert, unweighted
 *   forward (latent, width L):
 *            z    = Wd x                              bf16 [L][H], fp32 result
 *            acc  = sum_j w[j] * W2_e( act(W1_e z, W3_e z) )   router order;
 *                   the experts are [I][L] (W1, W3) and [L][I] (W2)
 *            acc  = acc * inv * gamma,  inv = 1/sqrt(sum(acc^2)/L + eps)
 *                   if latent_norm (the AGGREGATE is normed, not each expert)
 *            out  = Wu acc                            bf16 [H][L]
 *            out += S2( act(S1 x, S3 x) )             shared expert on the
 *                                                     ORIGINAL x, unweighted
 *   step (one decoder layer's MoE on the fp32 residual stream h):
 *            x    = bf16_RNE( h * inv * gamma ),  inv = fp32(1/sqrt(sum(h^2)/H + eps))
 *            h   += forward(x, route(x))          fp32, after the whole output
 *   act:     SiTU-GLU  b1*tanh(g/b1) * sigmoid(g) * b2*tanh(u/b2)   (default)
 *            SwiGLU    g * sigmoid(g) * u
 *
 * MXFP4 (README §4): weight = E2M1[nibble] * 2^(scale - 127); one E8M0
 * scale byte per 32 consecutive weights of a row; within a packed byte the
 * low nibble is the even-indexed weight; scale byte 255 makes its 32-group
 * contribute nothing; scale byte 0 is 2^-127.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define K3MOE_ABI_VERSION 3u

typedef enum {
    K3MOE_OK = 0,
    K3MOE_E_INVALID_ARG = 1,       /* NULL pointer, negative size, ...       */
    K3MOE_E_CONFIG = 2,            /* config field missing or out of range   */
    K3MOE_E_UNSUPPORTED_SHAPE = 3, /* a size the library's kernels refuse  */
    K3MOE_E_ALIGNMENT = 4,         /* a pointer or stride not 16-byte aligned */
    K3MOE_E_WORKSPACE = 5,         /* workspace NULL, too small or misaligned */
    K3MOE_E_OUT_OF_MEMORY = 6,     /* device memory could not be had         */
    K3MOE_E_HIP = 7                /* a HIP runtime call or launch failed    */
} k3moe_status;

typedef enum {
    K3MOE_ACT_SITU = 1,   /* SiTU-GLU with betas situ_b1, situ_b2 */
    K3MOE_ACT_SWIGLU = 2  /* g * sigmoid(g) * u                   */
} k3moe_act;              /* 0 is not a kind: an unset field is refused */

/* Layer configuration. No field has a default: every one must be set, and
 * struct_size / abi_version must equal sizeof(k3moe_config) and
 * K3MOE_ABI_VERSION (README §2 states the same refusal to guess for the
 * model's config). Supported sizes: hidden and inter positive multiples of
 * 128; shared_inter 0 (no shared expert) or a positive multiple of 128;
 * 1 <= topk <= n_experts <= 4096; latent 0 or a positive multiple of 128.
 * Two shared experts of width I_s each (the pages' n_shared = 2) are one
 * shared expert of width 2 I_s with their rows stacked (the activation is
 * elementwise, so the sum of the two is the stacked one). */
typedef struct {
    uint32_t struct_size;
    uint32_t abi_version;
    int32_t hidden;        /* H: token width                                */
    int32_t inter;         /* I: routed expert intermediate width           */
    int32_t n_experts;     /* E                                             */
    int32_t topk;          /* k                                             */
    int32_t shared_inter;  /* I_s of the one bf16 shared expert, 0 = none   */
    int32_t renorm;        /* 1: weights renormalised to sum 1; 0: not      */
    float routed_scale;    /* multiplies every routing weight (finite)      */
    int32_t act;           /* k3moe_act                                     */
    float situ_b1;         /* SiTU gate beta (> 0, finite; README uses 4)   */
    float situ_b2;         /* SiTU up beta   (> 0, finite; README uses 25)  */
    int32_t latent;        /* L: 0 = flat layer; > 0 = experts at width L   */
    int32_t latent_norm;   /* latent: 1 = RMSNorm on the aggregate, 0 = none;
                              flat: must be 0                               */
    float rms_eps;         /* latent_norm: epsilon inside the square root
                              (> 0, finite; README uses 1e-5); else ignored */
} k3moe_config;

/* One MXFP4 matrix per expert, E of them. Expert e's packed nibbles start
 * at packed + e * expert_stride_packed and are [rows][cols/2] bytes; its
 * scales start at scales + e * expert_stride_scales and are [rows][cols/32]
 * bytes. packed, scales and both strides must be multiples of 16; strides
 * must be at least the matrix size. */
typedef struct {
    const uint8_t *packed;
    const uint8_t *scales;
    int64_t expert_stride_packed;
    int64_t expert_stride_scales;
} k3moe_mxfp4;

/* The layer's weights (device pointers, caller-owned, never copied).
 * gate (W1) and up (W3) are [inter][hidden]; down (W2) is [hidden][inter].
 * router_w is bf16 [n_experts][hidden]; router_bias is fp32 [n_experts] or
 * NULL for no bias. Shared expert (bf16, NULL iff shared_inter == 0):
 * sh_gate and sh_up [shared_inter][hidden], sh_down [hidden][shared_inter].
 * Latent layer (latent = L > 0; all three NULL for a flat layer): lat_down
 * bf16 [L][hidden], lat_up bf16 [hidden][L], lat_norm fp32 [L] (the norm's
 * gamma; NULL iff latent_norm == 0); the experts' gate and up are then
 * [inter][L] and down [L][inter].
 * bf16 tensors are uint16 bit patterns; all bases 16-byte aligned. */
typedef struct {
    const uint16_t *router_w;
    const float *router_bias;
    k3moe_mxfp4 gate, up, down;
    const uint16_t *sh_gate, *sh_up, *sh_down;
    const uint16_t *lat_down, *lat_up;
    const float *lat_norm;
} k3moe_weights;

typedef struct k3moe_layer k3moe_layer;

/* Validate the config and weight descriptors and make a layer handle on the
 * current HIP device. The handle references the weights (it never copies or
 * repacks them) and owns one 8-byte device error counter. Checks that the
 * device has room for that counter plus a 1 MiB margin before allocating
 * (K3MOE_E_OUT_OF_MEMORY otherwise).
 *
 * Free device memory, here and in k3moe_cache_create, is hipMemGetInfo's
 * free bytes capped by the environment variable K3MOE_HBM_BUDGET (decimal
 * bytes) when it is set and non-empty: a process can hold the library to a
 * share of the device. A value that is not a plain decimal number (digits
 * only, below 2^64) gives K3MOE_E_INVALID_ARG. The kimi-k3-in-c README
 * (§11, streaming the trunk) adds up every allocation before making any;
 * both create calls do. */
k3moe_status k3moe_layer_create(const k3moe_config *cfg, const k3moe_weights *w,
                                k3moe_layer **out);

/* Bytes of workspace k3moe_route and k3moe_forward need for up to
 * max_tokens tokens (max_tokens >= 0). The caller allocates it (256-byte
 * aligned) and may reuse it across calls on one stream; calls in flight on
 * different streams need different workspaces. A batch is limited to
 * T*hidden*2 and T*topk*max(inter, shared_inter)*2 bytes below 2 GiB
 * (K3MOE_E_UNSUPPORTED_SHAPE above that; 43,690 tokens at hidden 7168,
 * top-16, inter 1536), here and in route/forward. */
k3moe_status k3moe_workspace_size(const k3moe_layer *layer, int32_t max_tokens,
                                  size_t *bytes);

/* Route T tokens (README §9, k3_router).
 *   x       bf16 [T][hidden]
 *   idx     int32 [T][topk]    out: selected experts, router order
 *   w       fp32  [T][topk]    out: routing weights
 *   logits  fp32  [T][n_experts] out (optional, NULL = not written): the
 *           fp32 logits the scores were taken from
 * T == 0 does nothing. */
k3moe_status k3moe_route(const k3moe_layer *layer, const uint16_t *x, int32_t T,
                         int32_t *idx, float *w, float *logits,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Expert layer for T tokens given their routes (README §9, k3_moe steps 3
 * and 6, flat).
 *   x    bf16  [T][hidden]
 *   idx  int32 [T][topk]   expert ids; an id outside [0, n_experts)
 *                          contributes nothing and is counted (see
 *                          k3moe_error_count), as the README counts dropped
 *                          experts instead of hiding them
 *   w    fp32  [T][topk]
 *   out  fp32  [T][hidden] out: written, not accumulated into (16-byte
 *                          aligned)
 * Deterministic: the same inputs give the same bits on every call; the
 * routed sum is taken in router order with no atomics. T == 0 does nothing. */
k3moe_status k3moe_forward(const k3moe_layer *layer, const uint16_t *x, int32_t T,
                           const int32_t *idx, const float *w, float *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Route and forward in one call: k3moe_route followed by k3moe_forward on
 * its routes (README §9: k3_router, then k3_moe), with the same arguments,
 * outputs and workspace. For one token of a flat layer (hidden <= 8192,
 * inter <= 2048, shared_inter <= 4096, topk <= 16) the whole layer runs in
 * three launches (router and shared gate/up; top-k, routed gate/up and
 * shared down; routed down and the router-order sum); other batches and
 * layers run route then forward. idx, w and out are written; logits as in
 * k3moe_route. Ids come from the router, so no drop can occur. The output
 * agrees with k3moe_forward on the same routes to the layer's error bound,
 * not bit for bit (the one-token kernels sum in another order). */
k3moe_status k3moe_route_forward(const k3moe_layer *layer, const uint16_t *x, int32_t T,
                                 int32_t *idx, float *w, float *logits, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* k3moe_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, bit for bit, with a fixed 64 MiB device array of the
 * library standing in for the workspace. Each GPU holds its own copy from the
 * moment the library is loaded there until the process ends. The call
 * allocates nothing (no hipMalloc, no event, no library allocation) and
 * takes no workspace argument.
 *   T whose workspace (k3moe_workspace_size) exceeds 64 MiB is refused with
 *   K3MOE_E_WORKSPACE before any launch (71 tokens at hidden 7168,
 *   top-16, inter 1536).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from different threads or layers) race.
 *   Serialise them on one stream. No part of the array has to start at zero.
 *   Per-stage profiling (k3moe_profile_enable) does not record these calls.
 * Other arguments and errors as k3moe_forward. */
k3moe_status k3moe_forward_noalloc(const k3moe_layer *layer, const uint16_t *x, int32_t T,
                                   const int32_t *idx, const float *w, float *out, void *stream);

/* k3moe_forward with the residual add fused into its last kernel, for a
 * stack of layers on an fp32 residual stream (each layer's output added to
 * the stream, the next layer reading it rounded to bf16):
 *   h  fp32 [T][hidden]  in/out, 16-byte aligned: h += forward(x, idx, w),
 *                        the complete layer output added once
 *   hb bf16 [T][hidden]  out (optional, NULL = not written): bf16_RNE of
 *                        the updated h; may be x itself (x is read before
 *                        the last kernel writes hb)
 * Other arguments and errors as k3moe_forward. */
k3moe_status k3moe_forward_residual(const k3moe_layer *layer, const uint16_t *x, int32_t T,
                                    const int32_t *idx, const float *w, float *h, uint16_t *hb,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* One decoder layer's MoE on the residual stream (README, the decoder-layer
 * listing after "Aggregate, attend, aggregate again": the layer input is
 * k3_rmsnorm of h with the post-attention gain, then k3_moe; the output is
 * added into the residual stream):
 *   x = bf16_RNE(h[t] * inv * gamma), inv = (float)(1 / sqrt(sum h^2 / H + eps))
 *       (README §5 k3_rmsnorm: fp64 sum of squares, epsilon inside the root,
 *       two fp32 products in that order; rounded once to bf16 because the
 *       layer takes bf16 tokens)
 *   idx, w = route(x)               as k3moe_route
 *   h[t] += forward(x, idx, w)      fp32, the complete layer output added once
 *   h      fp32 [T][hidden]  in/out, 16-byte aligned
 *   gamma  fp32 [hidden]     the norm's gain, 16-byte aligned
 *   eps    > 0 and finite, else K3MOE_E_INVALID_ARG
 *   x_out  bf16 [T][hidden]  out (optional, NULL = kept in the workspace): x
 *   idx    int32 [T][topk]   out
 *   w      fp32  [T][topk]   out
 *   hb     bf16 [T][hidden]  out (optional, NULL = not written):
 *                            bf16_RNE of the updated h
 * Uses the same workspace as route/forward (k3moe_workspace_size). Ids are
 * those of the router, so no drop can occur. T == 0 does nothing. */
k3moe_status k3moe_step(const k3moe_layer *layer, float *h, int32_t T, const float *gamma,
                        float eps, uint16_t *x_out, int32_t *idx, float *w, uint16_t *hb,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Number of (token, slot) assignments with an out-of-range expert id seen by
 * k3moe_forward since create or the last reset. Synchronises the stream. */
k3moe_status k3moe_error_count(const k3moe_layer *layer, uint64_t *n, void *stream);
k3moe_status k3moe_error_reset(k3moe_layer *layer, void *stream);

/* Per-stage timing on the caller's stream. While enabled, route, forward and step
 * record a HIP event pair around each of their kernel launches (stages
 * below); k3moe_profile_read synchronises the stream, returns per stage the
 * summed elapsed milliseconds and the number of launches since the last
 * read, and clears the record. Recording adds two event records per launch
 * to the stream, so time the layer itself with profiling off. */
typedef enum {
    K3MOE_STAGE_ROUTER = 0,         /* router logits, scores (one token of a flat layer:
                                       with the shared expert's gate/up rows) */
    K3MOE_STAGE_TOPK = 1,           /* top-k, weights (one token: inside GATEUP) */
    K3MOE_STAGE_PERM = 2,           /* token -> expert permutation        */
    K3MOE_STAGE_GATEUP = 3,         /* routed gate/up MXFP4 + activation  */
    K3MOE_STAGE_SHARED_GATEUP = 4,  /* shared expert gate/up + activation */
    K3MOE_STAGE_DOWN = 5,           /* down MXFP4 (+ shared down; one token: + the sum) */
    K3MOE_STAGE_COMBINE = 6,        /* router-order weighted sum + shared */
    K3MOE_STAGE_LATENT_IN = 7,      /* latent: down-projection of x       */
    K3MOE_STAGE_LATENT_OUT = 8,     /* latent: norm and up-projection     */
    K3MOE_STAGE_PRENORM = 9,        /* step: norm of the residual stream  */
    K3MOE_STAGE_CACHE_PLAN = 10,    /* cache: hits, victims, slot ids     */
    K3MOE_STAGE_CACHE_FILL = 11,    /* cache: host -> HBM expert reads    */
    K3MOE_STAGE_GATEUP_TILES = 12,  /* the routed gate/up tile GEMMs only (within GATEUP) */
    K3MOE_STAGE_DOWN_TILES = 13,    /* the routed down tile GEMMs only (within DOWN)      */
    K3MOE_N_STAGES = 14
} k3moe_stage;

k3moe_status k3moe_profile_enable(k3moe_layer *layer, int enable);
k3moe_status k3moe_profile_read(k3moe_layer *layer, double *ms, int64_t *launches,
                                int32_t n_stages, void *stream);

/* Experts beyond HBM: an arena of expert slots in HBM fed from host memory
 * (README §12 "An LRU cache for the experts"; the Kimi-K3.cpp README, "The
 * consumer-memory idea").
 *
 * The layer's routed expert tensors (gate, up, down: packed and scales) may
 * live in host memory: pinned pages the device can read (hipHostMalloc), or
 * device memory. The cache holds n_slots experts in HBM. Each
 * k3moe_cache_forward call, in stream order on the device:
 *   1. lists the distinct experts of idx in order of first appearance in the
 *      (token, slot) assignments;
 *   2. pins every one already resident (a hit) and stamps it as used;
 *   3. gives each miss, in that order, a victim slot: an empty slot (lowest
 *      index) if any, else the least recently used slot that is not pinned
 *      or already reserved in this call (ties: lowest index); a miss with no
 *      such slot left is dropped (its assignments contribute nothing and are
 *      counted in k3moe_error_count and in the cache's `dropped`);
 *   4. reads each reserved expert's six tensors from host memory into its
 *      slot, then runs the layer's expert kernels on the slots (k3moe_forward
 *      semantics: router-order sum, shared expert; `out` written).
 * The result is bit-identical to k3moe_forward on the same inputs when no
 * request is dropped. Calls on one cache must be serialised on one stream
 * (the slot table lives on the device and each call updates it). */
typedef struct k3moe_cache k3moe_cache;

typedef struct {
    uint64_t steps;          /* k3moe_cache_forward calls with T > 0        */
    uint64_t requests;       /* distinct experts asked for, summed          */
    uint64_t resident_hits;  /* of those, in a slot when the call began     */
    uint64_t misses;         /* of those, read from host memory             */
    uint64_t evictions;      /* misses that displaced a resident expert     */
    uint64_t dropped;        /* requests left without a slot                */
    uint64_t bytes_read;     /* host -> HBM expert bytes                    */
} k3moe_cache_stats;

/* n_slots in [1, n_experts]. Allocates the arena (n_slots times the
 * expert's six tensors, each 256-byte aligned) and the slot table; every
 * slot starts empty. The layer must outlive the cache. Returns
 * K3MOE_E_INVALID_ARG if an expert tensor is in host memory the device
 * cannot read (pageable memory), K3MOE_E_OUT_OF_MEMORY if the arena and
 * table (k3moe_cache_device_bytes) plus 1 MiB exceed the free device memory
 * (capped by K3MOE_HBM_BUDGET, see k3moe_layer_create); nothing is
 * allocated then. */
k3moe_status k3moe_cache_create(const k3moe_layer *layer, int32_t n_slots, k3moe_cache **out);

/* Device bytes k3moe_cache_create allocates for a layer of this config and
 * n_slots slots (the arena and the slot table), from the config alone (no
 * device call): what to budget before creating the cache. The create call
 * also keeps a 1 MiB margin free. Returns the config's refusal, or
 * K3MOE_E_INVALID_ARG for n_slots outside [1, n_experts]. */
k3moe_status k3moe_cache_device_bytes(const k3moe_config *cfg, int32_t n_slots, size_t *bytes);

/* Workspace bytes of k3moe_cache_forward for up to max_tokens tokens (also
 * enough for k3moe_route and k3moe_forward of the cache's layer). */
k3moe_status k3moe_cache_workspace_size(const k3moe_cache *cache, int32_t max_tokens, size_t *bytes);

/* The layer's expert forward through the cache (steps above).
 *   x bf16 [T][hidden], idx int32 [T][topk] (expert ids), w fp32 [T][topk],
 *   out fp32 [T][hidden] (16-byte aligned), written. T == 0 does nothing. */
k3moe_status k3moe_cache_forward(k3moe_cache *cache, const uint16_t *x, int32_t T,
                                 const int32_t *idx, const float *w, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Counters since create or the last reset. Synchronises the stream. */
k3moe_status k3moe_cache_stats_read(const k3moe_cache *cache, k3moe_cache_stats *stats, void *stream);

/* Which expert each slot holds (-1: empty), host int32 [n_slots].
 * Synchronises the stream. */
k3moe_status k3moe_cache_slots(const k3moe_cache *cache, int32_t *slots, void *stream);

/* Empties every slot and zeroes the counters (a kernel on the stream). */
k3moe_status k3moe_cache_reset(k3moe_cache *cache, void *stream);

/* Frees the arena and table (synchronises the device first). NULL is
 * accepted. */
void k3moe_cache_destroy(k3moe_cache *cache);

/* Frees the handle and its error counter (synchronises the device first).
 * NULL is accepted. */
void k3moe_layer_destroy(k3moe_layer *layer);

const char *k3moe_status_string(k3moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* K3MOE_H */
