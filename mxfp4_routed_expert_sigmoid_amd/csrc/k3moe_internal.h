// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "k3moe.h"

namespace k3moe {

// Activation split widths (number of e4m3 terms in the fp8 expansion that
// feeds the scaled MFMA's B operand): 4 for the fp32 expert activation (and
// for the single-token kernels' bf16 token).
constexpr int kATerms = 4;
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopk = 64;
// Tokens per chunk in the token -> expert permutation.
constexpr int kPermChunk = 16;

// Byte offsets of the workspace regions for T tokens (all 256-aligned).
struct WsLayout {
    size_t sc, ch;            // router scores, fp32 [T][E] each
    size_t rt_part;           // batched router fp64 partial sums [slices][T][E]
    size_t chunk_cnt;         // int32 [nchunks][E]
    size_t active_n;          // int32 [1]
    size_t active_e;          // int32 [E]
    size_t active_off;        // int32 [E + 1]
    size_t sorted;            // int32 [T * k]
    size_t act;               // routed activations, 4 bytes per element [T*k][I]:
                              //   fp32 (one token), or bf16 hi then bf16 lo planes
    size_t ash;               // shared activations, 4 bytes per element [T][I_s], same forms
    size_t sh_part;           // shared gate/up fp32 slice sums [slices][T][2][I_s] (small batches)
    size_t ys;                // expert outputs fp32 [T][k + 1][H] (slot k: shared expert)
    size_t tiles_gu, tiles_dn;  // grouped-GEMM tile lists, int2 each
    size_t light;             // int32 [4][E]: experts for the weight-streaming kernels (gate/up, down,
                              //   gate/up with one assignment, with two)
    size_t tile_n;            // int32 [6]: gate/up tiles, down tiles, light gate/up, light down,
                              //   light gate/up with one assignment, with two
    // f8 down tiles: the routed activation as n e4m3 terms [T*k][n][I] and
    // their E8M0 bytes [T*k][n][I/32] (the tiles write n = 3; sized for
    // kATerms)
    size_t aq = 0, aqs = 0;
    // latent layer only (0 otherwise)
    size_t lat_z = 0;         // z = Wd x as bf16 hi then lo planes [T][L] (4 bytes per element)
    size_t lat_acc = 0;       // routed aggregate fp32 [T][L]
    size_t lat_n = 0;         // normed aggregate as bf16 hi then lo planes [T][L]
    size_t lat_ysh = 0;       // shared expert output fp32 [T][H]
    size_t lat_part = 0;      // projection partial sums fp32 [slices][T][rows]
    size_t step_x = 0;        // k3moe_step: the normed bf16 tokens [T][H]
    size_t total;
};

WsLayout ws_layout(const k3moe_config &c, int64_t T);

struct LayerView {
    int H, I, E, K, Is;
    int renorm, act;
    float routed_scale, b1, b2;
    const uint16_t *router_w;
    const float *router_bias;
    const uint8_t *gp, *gs, *up, *us, *dp, *ds;
    int64_t g_sp, g_ss, u_sp, u_ss, d_sp, d_ss;
    const uint16_t *sh_gate, *sh_up, *sh_down;
    int Lt, EK;               // latent width (0: flat); the width the experts run at
    int lat_norm_on;
    float lat_eps;
    const uint16_t *lat_down, *lat_up;
    const float *lat_norm;
    unsigned long long *errors;
    bool routes_distinct = false;  // the ids come from the router (no expert twice in a token)
};

// Event pairs around kernel launches, per stage (k3moe_profile_*).
struct Profiler {
    bool on = false;
    struct Rec {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<hipEvent_t> spare;
    std::vector<Rec> recs;
    hipEvent_t take()
    {
        if (!spare.empty()) {
            hipEvent_t e = spare.back();
            spare.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};

// Brackets one stage's launches with an event pair when profiling is on.
struct StageMark {
    Profiler *p;
    int stage;
    hipStream_t s;
    hipEvent_t a = nullptr;
    StageMark(Profiler *p_, int stage_, hipStream_t s_) : p(p_), stage(stage_), s(s_)
    {
        if (p && p->on && (a = p->take())) (void)hipEventRecord(a, s);
    }
    ~StageMark()
    {
        if (!a) return;
        hipEvent_t b = p->take();
        if (!b) {
            p->spare.push_back(a);
            return;
        }
        (void)hipEventRecord(b, s);
        p->recs.push_back({stage, a, b});
    }
};

// Launchers (kernels live in k3moe_kernels.hip). Each returns the status of
// hipGetLastError() after its launches.
// Batched router (T > kRouterWaveMaxT): hidden-dimension slices and their width.
constexpr int kRouterWaveMaxT = 4;
int router_splits(int64_t T, int E, int H);
int router_kspan(int H, int S);

hipError_t launch_route(const LayerView &L, const uint16_t *x, int T, int32_t *idx,
                        float *w, float *logits, char *ws, const WsLayout &lay,
                        hipStream_t s, Profiler *prof);
hipError_t launch_topk(const LayerView &L, int T, const float *sc, const float *ch, int32_t *idx, float *w,
                       hipStream_t s);
hipError_t launch_router_t1(const LayerView &L, const uint16_t *x, float *sc, float *ch, float *logits,
                            hipStream_t s);
// What the layer's last kernel does with a result v of out[t][o]: store it
// (resid = false) or add it to the value already there (out += v, fp32, the
// residual stream); ob, when set, also receives bf16_RNE of the stored value.
struct OutEpi {
    bool resid = false;
    uint16_t *ob = nullptr;
};

hipError_t launch_forward(const LayerView &L, const uint16_t *x, int T,
                          const int32_t *idx, const float *w, float *out, char *ws,
                          const WsLayout &lay, hipStream_t s, Profiler *prof, const OutEpi &epi = OutEpi());

// The one-token layer in three launches (k3moe_decode.hip): route (when
// `route`; else idx/w are read) + experts + router-order combine into out
// with the epilogue. decode_fused_ok: the shapes it takes.
bool decode_fused_ok(const LayerView &L);
// routed: the router's scores are already in the workspace (sc, ch) and
// only the top-k and the experts run.
hipError_t launch_decode_fused(const LayerView &L, const uint16_t *x, int32_t *idx, float *w, float *logits,
                               bool route, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                               Profiler *prof, const OutEpi &epi = OutEpi(), bool routed = false);

// Gate/up of a batch's light experts that hold nt (1 or 2) assignments each
// (k3moe_decode.hip): items[0 .. *items_n) are active-list positions; the
// activation goes to act_hi/act_lo rows (the assignment's position), as the
// streamed gate/up writes it. gu_one_ok: the shapes it takes.
bool gu_one_ok(const LayerView &L);
hipError_t launch_gu_one(const LayerView &L, const uint16_t *x, int T, int nt, const int32_t *active_e,
                         const int32_t *active_off, const int32_t *sorted, const int32_t *items,
                         const int32_t *items_n, uint16_t *act_hi, uint16_t *act_lo, hipStream_t s);

// Expert slot cache (k3moe_cache.hip). Device counters, in this order:
enum {
    kCtrTick = 0,      // last use stamp handed out
    kCtrSteps,         // plans run
    kCtrRequests,      // distinct experts asked for
    kCtrHits,          // of those, resident when the plan began
    kCtrMisses,        // read into a slot
    kCtrEvictions,     // misses that displaced a resident expert
    kCtrDropped,       // requests that found no slot
    kCtrBytes,         // bytes read from host memory
    kCtrCount = 16
};
constexpr int kCacheSlotBits = 13;           // slot index bits of a victim key (slots <= 4096)
constexpr int64_t kFillChunk = 256 * 1024;   // bytes per fill block

struct CachePlanParams {
    const int32_t *idx;  // assignments [n] (expert ids)
    int64_t n;
    int E, S;
    int64_t expert_bytes;
    int32_t *slot_of;    // [E] device table
    int32_t *key_of;     // [S]
    long long *used_at;  // [S]
    unsigned long long *ctr;
    int32_t *remap;      // [n] out: slot ids
    int2 *fill;          // [S] out: (expert, slot)
    int32_t *nfill;      // out
};
struct CacheFillParams {
    const int2 *fill;
    const int32_t *nfill;
    const uint8_t *src[6];     // device-visible base of each tensor (expert 0)
    int64_t src_stride[6];     // bytes between experts
    int64_t seg_len[6];        // bytes per expert
    int64_t seg_off[6];        // offset in a slot
    uint8_t *arena;
    int64_t slot_bytes, expert_bytes;
    int nchunk;
};
size_t cache_plan_lds_bytes(int E, int S);
hipError_t launch_cache_init(unsigned long long *ctr, int32_t *slot_of, int E, int32_t *key_of, long long *used_at,
                             int S, hipStream_t s);
hipError_t launch_cache_plan_fill(const CachePlanParams &pp, const CacheFillParams &fp, int max_fill,
                                  hipStream_t s, Profiler *prof);

// Pre-MoE norm (k3moe_step.hip): x[t] = bf16_RNE(RMSNorm(h[t]) * gamma).
hipError_t launch_prenorm(const float *h, int T, int H, const float *gamma, float eps, uint16_t *x, hipStream_t s);
// The same norm and the one-token router (scores sc, ch) in one launch, T = 1.
bool prenorm_router_ok(const LayerView &L);
hipError_t launch_prenorm_router(const LayerView &L, const float *h, const float *gamma, float eps, uint16_t *x,
                                 float *sc, float *ch, hipStream_t s);

// A latent layer's experts for one token on the single-token kernels
// (k3moe_kernels.hip): routed rows (width EK) to the staging rows ys, the
// shared expert's rows to ysh [H].
bool latent_t1_ok(const LayerView &L);
hipError_t launch_latent_t1(const LayerView &L, const uint16_t *x, const uint16_t *zh, const uint16_t *zl,
                            const int32_t *idx, float *act, float *ash, char *ys_base, float *ysh, hipStream_t s,
                            Profiler *prof);

// Latent layer (k3moe_latent.hip): projections with bf16 weights, the norm.
int proj_splits(int64_t T, int R, int Kd);
hipError_t launch_latent_forward(const LayerView &L, const uint16_t *x, int T, const int32_t *idx,
                                 const float *w, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                                 Profiler *prof, const OutEpi &epi);

// Grouped GEMMs for batches (k3moe_grouped.hip).
size_t grouped_tile_cap_gu(int64_t T, int K, int E);
size_t grouped_tile_cap_dn(int64_t T, int K, int E);
// xr: the routed experts' tokens, bf16 [T][EK] (x for a flat layer); xr_lo:
// a second plane (lo of an fp32 input) or null. ysh: the shared expert's
// output fp32 [T][H], or null for slot k of ys. Routed outputs go to ys
// [T][k + 1][EK].
// term buffers of the f8 down tiles (null: those tiles run on bf16)
struct TermBufs {
    uint8_t *aq = nullptr, *aqs = nullptr;   // the routed activation's terms
};
// The term regions of a workspace.
inline TermBufs term_bufs(char *ws, const WsLayout &lay)
{
    TermBufs t;
    t.aq = reinterpret_cast<uint8_t *>(ws + lay.aq);
    t.aqs = reinterpret_cast<uint8_t *>(ws + lay.aqs);
    return t;
}
hipError_t launch_grouped(const LayerView &L, const uint16_t *x, const uint16_t *xr, const uint16_t *xr_lo, int T,
                          const int32_t *active_n, const int32_t *active_e, const int32_t *active_off,
                          const int32_t *sorted, uint16_t *act_hi, uint16_t *act_lo, uint16_t *ash_hi,
                          uint16_t *ash_lo, float *sh_part, int2 *tiles_gu, int2 *tiles_dn, int32_t *light,
                          int32_t *counts, float *ys, float *ysh, hipStream_t s, Profiler *prof,
                          const TermBufs &tb = TermBufs());

// Weight-streaming kernels for experts with few tokens (k3moe_stream.hip).
bool stream_path_ok(const LayerView &L);
bool stream_down_ok(const LayerView &L, int T);
int stream_max_tokens();
int stream_shared_slices(int T);
bool stream_shared_ok(const LayerView &L, int T);
int stream_shared_down_slices(int Lt, int Is, int T, int I);
int stream_down_rows(const LayerView &L, int T);
hipError_t launch_stream_gu(const LayerView &L, const uint16_t *x, const uint16_t *xr, const uint16_t *xr_lo,
                            int T, const int32_t *active_e, const int32_t *active_off, const int32_t *sorted,
                            const int32_t *light, const int32_t *light_n, bool with_shared, uint16_t *act_hi,
                            uint16_t *act_lo, uint16_t *ash_hi, uint16_t *ash_lo, float *sh_part, hipStream_t s);
hipError_t launch_stream_dn(const LayerView &L, int T, const int32_t *active_e, const int32_t *active_off,
                            const int32_t *sorted, const int32_t *light, const int32_t *light_n,
                            bool with_shared, const uint16_t *act_hi, const uint16_t *act_lo,
                            const uint16_t *ash_hi, const uint16_t *ash_lo, float *ys, float *ysh, hipStream_t s);

// Token -> expert permutation and router-order combine (k3moe_kernels.hip).
void launch_perm(const LayerView &L, const int32_t *idx, int T, char *ws, const WsLayout &lay, hipStream_t s,
                 Profiler *prof);
void launch_combine(const LayerView &L, const float *ys, const float *w, const int32_t *idx, int T, int width,
                    bool shared, float *out, hipStream_t s, const OutEpi &epi = OutEpi());

}  // namespace k3moe
