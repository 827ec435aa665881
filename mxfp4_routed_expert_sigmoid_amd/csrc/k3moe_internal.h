// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "k3moe.h"

namespace k3moe {

// Activation split widths (number of e4m3 terms in the fp8 expansion that
// feeds the scaled MFMA's B operand): 4 for a bf16 token vector (exact) and
// 4 for the fp32 expert activation.
constexpr int kXTerms = 4;
constexpr int kATerms = 4;
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopk = 64;
// Tokens per chunk in the token -> expert permutation.
constexpr int kPermChunk = 16;

// Byte offsets of the workspace regions for T tokens (all 256-aligned).
struct WsLayout {
    size_t sc, ch;            // router scores, fp32 [T][E] each
    size_t xq, xs;            // token fp8 terms [T][3][H], scales [T][3][H/32]
    size_t chunk_cnt;         // int32 [nchunks][E]
    size_t active_n;          // int32 [1]
    size_t active_e;          // int32 [E]
    size_t active_off;        // int32 [E + 1]
    size_t sorted;            // int32 [T * k]
    size_t aq, as;            // activation fp8 terms [T*k][4][I], scales [T*k][4][I/32]
    size_t ash;               // shared activation fp32 [T][I_s]
    size_t ys;                // expert outputs fp32 [T][k + 1][H] (slot k: shared expert)
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
    unsigned long long *errors;
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
hipError_t launch_route(const LayerView &L, const uint16_t *x, int T, int32_t *idx,
                        float *w, float *logits, char *ws, const WsLayout &lay,
                        hipStream_t s, Profiler *prof);
hipError_t launch_forward(const LayerView &L, const uint16_t *x, int T,
                          const int32_t *idx, const float *w, float *out, char *ws,
                          const WsLayout &lay, hipStream_t s, Profiler *prof);

}  // namespace k3moe
