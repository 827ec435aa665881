// C-ABI entry points of libk3moe: argument validation, workspace layout,
// launches on the caller's stream. See include/k3moe.h for the contract.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "k3moe_internal.h"

struct k3moe_layer {
    k3moe_config cfg;
    k3moe_weights w;
    int device;
    unsigned long long *errors;  // device counter of out-of-range expert ids
    k3moe::Profiler *prof;       // per-stage event timing (k3moe_profile_*)
};

struct k3moe_cache {
    const k3moe_layer *layer;
    int S;                       // slots
    int device;
    const uint8_t *src[6];       // device-visible expert tensors: gate, up, down (packed, scales)
    int64_t src_stride[6];
    int64_t seg_len[6], seg_off[6];
    int64_t slot_bytes, expert_bytes;
    uint8_t *arena;              // [S][slot_bytes]
    char *table;                 // counters, slot_of [E], key_of [S], used_at [S]
    unsigned long long *ctr;
    int32_t *slot_of, *key_of;
    long long *used_at;
};

namespace k3moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const k3moe_config &c, int64_t T)
{
    const int64_t H = c.hidden, I = c.inter, E = c.n_experts, K = c.topk, Is = c.shared_inter;
    const int64_t Lt = c.latent, EK = Lt ? Lt : H;
    const int64_t nchunks = std::max<int64_t>(1, (T + kPermChunk - 1) / kPermChunk);
    WsLayout L;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + std::max<size_t>(bytes, 1));
        return at;
    };
    L.sc = take(sizeof(float) * T * E);
    L.ch = take(sizeof(float) * T * E);
    {
        // a call may take fewer tokens than the workspace was sized for, and
        // the slice count falls as T grows: the largest partial buffer over
        // every T' <= T (no batch of more than 128 * 512 tokens is sliced: 512 tiles of 128)
        size_t part = 0;
        for (int64_t t = kRouterWaveMaxT + 1; t <= std::min<int64_t>(T, 128 * 512); ++t) {
            const int S = router_splits(t, (int)E, (int)H);
            if (S > 1) part = std::max(part, sizeof(double) * S * t * E);
        }
        L.rt_part = take(part);
    }
    L.chunk_cnt = take(sizeof(int32_t) * nchunks * E);
    L.active_n = take(sizeof(int32_t));
    L.active_e = take(sizeof(int32_t) * E);
    L.active_off = take(sizeof(int32_t) * (E + 1));
    L.sorted = take(sizeof(int32_t) * std::max<int64_t>(1, T * K));
    L.act = take((size_t)T * K * 4 * I);
    L.ash = take(sizeof(float) * T * std::max<int64_t>(Is, 1));
    L.ys = take(sizeof(float) * T * (K + 1) * std::max(H, EK));
    {
        // the slice count is non-increasing in T: the largest buffer over T' <= T
        size_t part = 0;
        for (int64_t t = 1; t <= std::min<int64_t>(T, 4096); ++t) {  // one token too: the grouped path can take it
            const int S = stream_shared_slices((int)t);
            if (S > 1) part = std::max(part, sizeof(float) * S * t * 2 * Is);
        }
        L.sh_part = take(part);
    }
    L.tiles_gu = take(sizeof(int2) * grouped_tile_cap_gu(T, (int)K, (int)E));
    L.tiles_dn = take(sizeof(int2) * grouped_tile_cap_dn(T, (int)K, (int)E));
    L.light = take(sizeof(int32_t) * 4 * E);
    L.tile_n = take(6 * sizeof(int32_t));
    L.aq = take((size_t)T * K * kATerms * I);
    L.aqs = take((size_t)T * K * kATerms * (I / 32));
    if (Lt > 0) {
        L.lat_z = take((size_t)T * Lt * 4);
        L.lat_acc = take(sizeof(float) * T * Lt);
        L.lat_n = take((size_t)T * Lt * 4);
        // the shared expert's output, in K-slice partial sums for a few tokens
        size_t ysh = sizeof(float) * T * H;
        for (int64_t t = 1; t <= std::min<int64_t>(T, 128); ++t)  // the streamed shared expert: T <= 128
            ysh = std::max(ysh, sizeof(float) * stream_shared_down_slices((int)Lt, (int)Is, (int)t, (int)I) * t * H);
        L.lat_ysh = take(ysh);
        // projection partial sums: the largest over T' <= T of either projection
        // (one slice at least: the projections always sum through them)
        size_t part = sizeof(float) * T * std::max(Lt, H);
        for (int64_t t = 1; t <= std::min<int64_t>(T, 4096); ++t) {
            const int Sd = proj_splits(t, (int)Lt, (int)H), Su = proj_splits(t, (int)H, (int)Lt);
            if (Sd > 1) part = std::max(part, sizeof(float) * Sd * t * Lt);
            if (Su > 1) part = std::max(part, sizeof(float) * Su * t * H);
        }
        L.lat_part = take(part);
    }
    L.step_x = take((size_t)T * H * 2);
    L.total = o;
    return L;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static k3moe_status check_config(const k3moe_config *c)
{
    if (!c) return K3MOE_E_INVALID_ARG;
    if (c->struct_size != sizeof(k3moe_config) || c->abi_version != K3MOE_ABI_VERSION)
        return K3MOE_E_CONFIG;
    if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0 || c->topk <= 0 || c->shared_inter < 0)
        return K3MOE_E_CONFIG;
    if (c->topk > c->n_experts) return K3MOE_E_CONFIG;
    if (c->renorm != 0 && c->renorm != 1) return K3MOE_E_CONFIG;
    if (c->act != K3MOE_ACT_SITU && c->act != K3MOE_ACT_SWIGLU) return K3MOE_E_CONFIG;
    if (!isfinite(c->routed_scale)) return K3MOE_E_CONFIG;
    if (c->act == K3MOE_ACT_SITU &&
        !(isfinite(c->situ_b1) && isfinite(c->situ_b2) && c->situ_b1 > 0.0f && c->situ_b2 > 0.0f))
        return K3MOE_E_CONFIG;
    if (c->hidden % 128 || c->inter % 128 || c->shared_inter % 128) return K3MOE_E_UNSUPPORTED_SHAPE;
    if (c->n_experts > kMaxExperts || c->topk > kMaxTopk) return K3MOE_E_UNSUPPORTED_SHAPE;
    if (c->latent < 0) return K3MOE_E_CONFIG;
    if (c->latent == 0) {
        if (c->latent_norm != 0) return K3MOE_E_CONFIG;
    } else {
        if (c->latent_norm != 0 && c->latent_norm != 1) return K3MOE_E_CONFIG;
        if (c->latent_norm && !(isfinite(c->rms_eps) && c->rms_eps > 0.0f)) return K3MOE_E_CONFIG;
        if (c->latent % 128) return K3MOE_E_UNSUPPORTED_SHAPE;
    }
    // 32-bit row/element indexing inside the kernels
    const int64_t ek = c->latent ? c->latent : c->hidden;
    if ((int64_t)c->hidden * c->inter > (int64_t)1 << 30 || ek * c->inter > (int64_t)1 << 30 ||
        ek * c->hidden > (int64_t)1 << 30)
        return K3MOE_E_UNSUPPORTED_SHAPE;
    return K3MOE_OK;
}

static k3moe_status check_mxfp4(const k3moe_mxfp4 &m, int64_t rows, int64_t cols, int64_t E)
{
    if (!m.packed || !m.scales) return K3MOE_E_INVALID_ARG;
    const int64_t pbytes = rows * cols / 2, sbytes = rows * cols / 32;
    if (E > 1 && (m.expert_stride_packed < pbytes || m.expert_stride_scales < sbytes))
        return K3MOE_E_INVALID_ARG;
    if (!aligned(m.packed, 16) || m.expert_stride_packed % 16) return K3MOE_E_ALIGNMENT;
    if (!aligned(m.scales, 16) || m.expert_stride_scales % 16) return K3MOE_E_ALIGNMENT;
    return K3MOE_OK;
}

static k3moe_status check_weights(const k3moe_config *c, const k3moe_weights *w)
{
    if (!w) return K3MOE_E_INVALID_ARG;
    if (!w->router_w) return K3MOE_E_INVALID_ARG;
    if (!aligned(w->router_w, 16) || (w->router_bias && !aligned(w->router_bias, 4)))
        return K3MOE_E_ALIGNMENT;
    k3moe_status s;
    const int64_t ek = c->latent ? c->latent : c->hidden;  // width the experts run at
    if ((s = check_mxfp4(w->gate, c->inter, ek, c->n_experts)) != K3MOE_OK) return s;
    if ((s = check_mxfp4(w->up, c->inter, ek, c->n_experts)) != K3MOE_OK) return s;
    if ((s = check_mxfp4(w->down, ek, c->inter, c->n_experts)) != K3MOE_OK) return s;
    if (c->latent == 0) {
        if (w->lat_down || w->lat_up || w->lat_norm) return K3MOE_E_INVALID_ARG;
    } else {
        if (!w->lat_down || !w->lat_up || (c->latent_norm ? !w->lat_norm : w->lat_norm != nullptr))
            return K3MOE_E_INVALID_ARG;
        if (!aligned(w->lat_down, 16) || !aligned(w->lat_up, 16) || (w->lat_norm && !aligned(w->lat_norm, 16)))
            return K3MOE_E_ALIGNMENT;
    }
    const bool any = w->sh_gate || w->sh_up || w->sh_down;
    const bool all = w->sh_gate && w->sh_up && w->sh_down;
    if (c->shared_inter == 0 ? any : !all) return K3MOE_E_INVALID_ARG;
    if (all && !(aligned(w->sh_gate, 16) && aligned(w->sh_up, 16) && aligned(w->sh_down, 16)))
        return K3MOE_E_ALIGNMENT;
    return K3MOE_OK;
}

static LayerView view(const k3moe_layer *l)
{
    const k3moe_config &c = l->cfg;
    const k3moe_weights &w = l->w;
    LayerView v;
    v.H = c.hidden;
    v.I = c.inter;
    v.E = c.n_experts;
    v.K = c.topk;
    v.Is = c.shared_inter;
    v.renorm = c.renorm;
    v.act = c.act;
    v.routed_scale = c.routed_scale;
    v.b1 = c.situ_b1;
    v.b2 = c.situ_b2;
    v.router_w = w.router_w;
    v.router_bias = w.router_bias;
    v.gp = w.gate.packed;
    v.gs = w.gate.scales;
    v.up = w.up.packed;
    v.us = w.up.scales;
    v.dp = w.down.packed;
    v.ds = w.down.scales;
    v.g_sp = w.gate.expert_stride_packed;
    v.g_ss = w.gate.expert_stride_scales;
    v.u_sp = w.up.expert_stride_packed;
    v.u_ss = w.up.expert_stride_scales;
    v.d_sp = w.down.expert_stride_packed;
    v.d_ss = w.down.expert_stride_scales;
    v.sh_gate = w.sh_gate;
    v.sh_up = w.sh_up;
    v.sh_down = w.sh_down;
    v.Lt = c.latent;
    v.EK = c.latent ? c.latent : c.hidden;
    v.lat_norm_on = c.latent ? c.latent_norm : 0;
    v.lat_eps = c.rms_eps;
    v.lat_down = w.lat_down;
    v.lat_up = w.lat_up;
    v.lat_norm = w.lat_norm;
    v.errors = l->errors;
    return v;
}

// The batched kernels address token rows, activation rows and staging rows
// with 32-bit byte offsets: a batch whose planes exceed 2 GiB is refused.
static bool batch_fits(const k3moe_config &c, int64_t T)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t I = std::max(c.inter, c.shared_inter);
    return T * c.hidden * 2 < lim && T * c.topk * I * 2 < lim;
}

// Free HBM as the library plans against it: hipMemGetInfo's free bytes,
// capped by K3MOE_HBM_BUDGET (decimal bytes) when that is set, so a process
// can keep the library inside a share of the device (and a test can stand in
// a shortfall). An unparsable value is refused.
static k3moe_status free_hbm(size_t *free_b)
{
    size_t total_b = 0;
    if (hipMemGetInfo(free_b, &total_b) != hipSuccess) return K3MOE_E_HIP;
    const char *env = std::getenv("K3MOE_HBM_BUDGET");
    if (env && *env) {
        // digits only (no sign, space or exponent), at most 2^64 - 1
        unsigned long long v = 0;
        for (const char *c = env; *c; ++c) {
            if (*c < '0' || *c > '9') return K3MOE_E_INVALID_ARG;
            const unsigned d = (unsigned)(*c - '0');
            if (v > (~0ull - d) / 10) return K3MOE_E_INVALID_ARG;
            v = v * 10 + d;
        }
        if (v < *free_b) *free_b = (size_t)v;
    }
    return K3MOE_OK;
}

// Device bytes a layer handle allocates (the error counter), and the margin
// every create call keeps free beyond its own allocations.
constexpr size_t kLayerDeviceBytes = sizeof(unsigned long long);
constexpr size_t kCreateMarginBytes = (size_t)1 << 20;

// The cache's device allocations, from the layer's config alone: per slot
// the expert's six tensors (gate, up, down; packed then scales), each
// 256-byte aligned, in that order; the table holds the counters, the expert
// -> slot map and the per-slot key and last use.
struct CachePlan {
    int64_t seg_len[6], seg_off[6];
    int64_t slot_bytes, expert_bytes;
    size_t arena, table;
};

static CachePlan cache_plan(const k3moe_config &c, int32_t n_slots)
{
    CachePlan p{};
    const int64_t EK = c.latent ? c.latent : c.hidden;
    const int64_t elems = (int64_t)c.inter * EK;  // every expert matrix has I * EK weights
    int64_t off = 0;
    for (int i = 0; i < 6; ++i) {
        p.seg_len[i] = (i & 1) ? elems / 32 : elems / 2;
        p.seg_off[i] = off;
        off = (int64_t)align256((size_t)(off + p.seg_len[i]));
        p.expert_bytes += p.seg_len[i];
    }
    p.slot_bytes = off;
    p.arena = (size_t)p.slot_bytes * (size_t)n_slots;
    p.table = align256(sizeof(unsigned long long) * kCtrCount) + align256(sizeof(int32_t) * c.n_experts) +
              align256(sizeof(int32_t) * n_slots) + align256(sizeof(long long) * n_slots);
    return p;
}

// Common checks of a route/forward call; T == 0 is reported as "nothing to do".
static k3moe_status check_call(const k3moe_layer *l, int32_t T, void *ws, size_t ws_bytes,
                               bool *nothing)
{
    *nothing = false;
    if (!l || T < 0) return K3MOE_E_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return K3MOE_E_HIP;
    if (dev != l->device) return K3MOE_E_INVALID_ARG;
    if (T == 0) {
        *nothing = true;
        return K3MOE_OK;
    }
    if (!batch_fits(l->cfg, T)) return K3MOE_E_UNSUPPORTED_SHAPE;
    if (!ws || !aligned(ws, 256)) return K3MOE_E_WORKSPACE;
    if (ws_bytes < ws_layout(l->cfg, T).total) return K3MOE_E_WORKSPACE;
    return K3MOE_OK;
}

// The layer as the expert kernels see it through a cache: S "experts" (the
// slots), each tensor at its offset in slot 0 with the slot stride.
static LayerView cache_view(const k3moe_cache *c)
{
    LayerView v = view(c->layer);
    v.E = c->S;
    const uint8_t **dst[6] = {&v.gp, &v.gs, &v.up, &v.us, &v.dp, &v.ds};
    for (int i = 0; i < 6; ++i) *dst[i] = c->arena + c->seg_off[i];
    v.g_sp = v.g_ss = v.u_sp = v.u_ss = v.d_sp = v.d_ss = c->slot_bytes;
    return v;
}

struct CacheWs {
    WsLayout lay;          // the layer's workspace at S experts
    size_t remap, fill, nfill, total;
};

static CacheWs cache_ws(const k3moe_cache *c, int64_t T)
{
    k3moe_config cs = c->layer->cfg;
    cs.n_experts = c->S;
    CacheWs w;
    w.lay = ws_layout(cs, T);
    size_t o = align256(w.lay.total);
    w.remap = o;
    o = align256(o + std::max<size_t>(sizeof(int32_t) * T * cs.topk, 1));
    w.fill = o;
    o = align256(o + sizeof(int2) * c->S);
    w.nfill = o;
    w.total = align256(o + sizeof(int32_t));
    return w;
}

// Allocation-free forward (k3moe_forward_noalloc): a fixed device array
// stands in for the caller's workspace. Each GPU the library runs on holds
// its own copy (a module global), so its address is looked up once per
// device, with that device current, when the first layer is created there.
// In host code the array's name is only a stand-in for the device symbol:
// kernels and copies take the looked-up address, never the name.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static char *g_scratch_ptr[kMaxScratchDevices];

static k3moe_status resolve_scratch(int dev)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return K3MOE_E_UNSUPPORTED_SHAPE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return K3MOE_OK;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return K3MOE_E_HIP;
    }
    g_scratch_ptr[dev] = static_cast<char *>(p);
    return K3MOE_OK;
}

static char *scratch_of(int dev)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[dev];
}

}  // namespace k3moe

using namespace k3moe;

extern "C" {

k3moe_status k3moe_layer_create(const k3moe_config *cfg, const k3moe_weights *w, k3moe_layer **out)
{
    if (!out) return K3MOE_E_INVALID_ARG;
    *out = nullptr;
    k3moe_status s = check_config(cfg);
    if (s != K3MOE_OK) return s;
    if ((s = check_weights(cfg, w)) != K3MOE_OK) return s;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return K3MOE_E_HIP;
    if ((s = resolve_scratch(dev)) != K3MOE_OK) return s;  // this device's k3moe_forward_noalloc scratch
    size_t free_b = 0;
    if ((s = free_hbm(&free_b)) != K3MOE_OK) return s;
    if (free_b < kLayerDeviceBytes + kCreateMarginBytes) return K3MOE_E_OUT_OF_MEMORY;
    k3moe_layer *l = new (std::nothrow) k3moe_layer;
    if (!l) return K3MOE_E_OUT_OF_MEMORY;
    l->cfg = *cfg;
    l->w = *w;
    l->device = dev;
    l->errors = nullptr;
    l->prof = new (std::nothrow) Profiler;
    if (!l->prof) {
        delete l;
        return K3MOE_E_OUT_OF_MEMORY;
    }
    if (hipMalloc(&l->errors, sizeof(unsigned long long)) != hipSuccess) {
        delete l->prof;
        delete l;
        return K3MOE_E_OUT_OF_MEMORY;
    }
    if (hipMemset(l->errors, 0, sizeof(unsigned long long)) != hipSuccess) {
        (void)hipFree(l->errors);
        delete l->prof;
        delete l;
        return K3MOE_E_HIP;
    }
    *out = l;
    return K3MOE_OK;
}

k3moe_status k3moe_workspace_size(const k3moe_layer *l, int32_t max_tokens, size_t *bytes)
{
    if (!l || !bytes || max_tokens < 0) return K3MOE_E_INVALID_ARG;
    if (!batch_fits(l->cfg, max_tokens)) return K3MOE_E_UNSUPPORTED_SHAPE;
    *bytes = ws_layout(l->cfg, max_tokens).total;
    return K3MOE_OK;
}

k3moe_status k3moe_route(const k3moe_layer *l, const uint16_t *x, int32_t T, int32_t *idx, float *w,
                         float *logits, void *ws, size_t ws_bytes, void *stream)
{
    bool nothing;
    k3moe_status s = check_call(l, T, ws, ws_bytes, &nothing);
    if (s != K3MOE_OK || nothing) return s;
    if (!x || !idx || !w) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4)))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    if (launch_route(view(l), x, T, idx, w, logits, static_cast<char *>(ws), lay,
                     static_cast<hipStream_t>(stream), l->prof) != hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_forward(const k3moe_layer *l, const uint16_t *x, int32_t T, const int32_t *idx,
                           const float *w, float *out, void *ws, size_t ws_bytes, void *stream)
{
    bool nothing;
    k3moe_status s = check_call(l, T, ws, ws_bytes, &nothing);
    if (s != K3MOE_OK || nothing) return s;
    if (!x || !idx || !w || !out) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(out, 16))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    if (launch_forward(view(l), x, T, idx, w, out, static_cast<char *>(ws), lay,
                       static_cast<hipStream_t>(stream), l->prof) != hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_route_forward(const k3moe_layer *l, const uint16_t *x, int32_t T, int32_t *idx, float *w,
                                 float *logits, float *out, void *ws, size_t ws_bytes, void *stream)
{
    bool nothing;
    k3moe_status s = check_call(l, T, ws, ws_bytes, &nothing);
    if (s != K3MOE_OK || nothing) return s;
    if (!x || !idx || !w || !out) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4)) ||
        !aligned(out, 16))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    char *wsc = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    LayerView v = view(l);
    if (T == 1 && decode_fused_ok(v)) {
        if (launch_decode_fused(v, x, idx, w, logits, true, out, wsc, lay, st, l->prof) != hipSuccess)
            return K3MOE_E_HIP;
        return K3MOE_OK;
    }
    v.routes_distinct = true;  // the routes below come from the router
    if (launch_route(v, x, T, idx, w, logits, wsc, lay, st, l->prof) != hipSuccess) return K3MOE_E_HIP;
    if (launch_forward(v, x, T, idx, w, out, wsc, lay, st, l->prof) != hipSuccess) return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_forward_noalloc(const k3moe_layer *l, const uint16_t *x, int32_t T, const int32_t *idx,
                                   const float *w, float *out, void *stream)
{
    if (!l) return K3MOE_E_INVALID_ARG;
    char *ws = scratch_of(l->device);
    if (!ws) return K3MOE_E_HIP;  // the layer's device has no resolved scratch
    bool nothing;
    k3moe_status s = check_call(l, T, ws, kScratchBytes, &nothing);  // T beyond the scratch: E_WORKSPACE
    if (s != K3MOE_OK || nothing) return s;
    if (!x || !idx || !w || !out) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(out, 16))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    // no profiler: its event records could create events
    if (launch_forward(view(l), x, T, idx, w, out, ws, lay, static_cast<hipStream_t>(stream), nullptr) !=
        hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_forward_residual(const k3moe_layer *l, const uint16_t *x, int32_t T, const int32_t *idx,
                                    const float *w, float *h, uint16_t *hb, void *ws, size_t ws_bytes,
                                    void *stream)
{
    bool nothing;
    k3moe_status s = check_call(l, T, ws, ws_bytes, &nothing);
    if (s != K3MOE_OK || nothing) return s;
    if (!x || !idx || !w || !h) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(h, 16) || (hb && !aligned(hb, 16)))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    OutEpi epi;
    epi.resid = true;
    epi.ob = hb;
    if (launch_forward(view(l), x, T, idx, w, h, static_cast<char *>(ws), lay, static_cast<hipStream_t>(stream),
                       l->prof, epi) != hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_step(const k3moe_layer *l, float *h, int32_t T, const float *gamma, float eps,
                        uint16_t *x_out, int32_t *idx, float *w, uint16_t *hb, void *ws, size_t ws_bytes,
                        void *stream)
{
    bool nothing;
    k3moe_status s = check_call(l, T, ws, ws_bytes, &nothing);
    if (s != K3MOE_OK || nothing) return s;
    if (!h || !gamma || !idx || !w || !(eps > 0.0f) || !std::isfinite(eps)) return K3MOE_E_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(gamma, 16) || !aligned(idx, 4) || !aligned(w, 4) ||
        (x_out && !aligned(x_out, 16)) || (hb && !aligned(hb, 16)))
        return K3MOE_E_ALIGNMENT;
    const WsLayout lay = ws_layout(l->cfg, T);
    char *wsc = static_cast<char *>(ws);
    uint16_t *x = x_out ? x_out : reinterpret_cast<uint16_t *>(wsc + lay.step_x);
    hipStream_t st = static_cast<hipStream_t>(stream);
    LayerView v = view(l);
    v.routes_distinct = true;  // the routes below come from the router
    OutEpi epi;
    epi.resid = true;
    epi.ob = hb;
    if (T == 1 && decode_fused_ok(v) && prenorm_router_ok(v)) {
        // the norm and the router in one launch, then the top-k and the experts
        {
            StageMark m(l->prof, K3MOE_STAGE_ROUTER, st);
            if (launch_prenorm_router(v, h, gamma, eps, x, reinterpret_cast<float *>(wsc + lay.sc),
                                      reinterpret_cast<float *>(wsc + lay.ch), st) != hipSuccess)
                return K3MOE_E_HIP;
        }
        if (launch_decode_fused(v, x, idx, w, nullptr, true, h, wsc, lay, st, l->prof, epi, true) != hipSuccess)
            return K3MOE_E_HIP;
        return K3MOE_OK;
    }
    {
        StageMark m(l->prof, K3MOE_STAGE_PRENORM, st);
        if (launch_prenorm(h, T, v.H, gamma, eps, x, st) != hipSuccess) return K3MOE_E_HIP;
    }
    if (launch_route(v, x, T, idx, w, nullptr, wsc, lay, st, l->prof) != hipSuccess) return K3MOE_E_HIP;
    if (launch_forward(v, x, T, idx, w, h, wsc, lay, st, l->prof, epi) != hipSuccess) return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_error_count(const k3moe_layer *l, uint64_t *n, void *stream)
{
    if (!l || !n) return K3MOE_E_INVALID_ARG;
    unsigned long long v = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&v, l->errors, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
        return K3MOE_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return K3MOE_E_HIP;
    *n = v;
    return K3MOE_OK;
}

k3moe_status k3moe_error_reset(k3moe_layer *l, void *stream)
{
    if (!l) return K3MOE_E_INVALID_ARG;
    if (hipMemsetAsync(l->errors, 0, sizeof(unsigned long long), static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_profile_enable(k3moe_layer *l, int enable)
{
    if (!l) return K3MOE_E_INVALID_ARG;
    l->prof->on = enable != 0;
    return K3MOE_OK;
}

k3moe_status k3moe_profile_read(k3moe_layer *l, double *ms, int64_t *launches, int32_t n_stages,
                                void *stream)
{
    if (!l || !ms || !launches || n_stages < 0) return K3MOE_E_INVALID_ARG;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return K3MOE_E_HIP;
    for (int i = 0; i < n_stages; ++i) {
        ms[i] = 0.0;
        launches[i] = 0;
    }
    Profiler &p = *l->prof;
    k3moe_status st = K3MOE_OK;
    for (const Profiler::Rec &r : p.recs) {
        float t = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            st = K3MOE_E_HIP;
        if (r.stage < n_stages) {
            ms[r.stage] += t;
            launches[r.stage] += 1;
        }
        p.spare.push_back(r.a);
        p.spare.push_back(r.b);
    }
    p.recs.clear();
    return st;
}

k3moe_status k3moe_cache_create(const k3moe_layer *l, int32_t n_slots, k3moe_cache **out)
{
    if (!out) return K3MOE_E_INVALID_ARG;
    *out = nullptr;
    if (!l || n_slots < 1 || n_slots > l->cfg.n_experts) return K3MOE_E_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return K3MOE_E_HIP;
    if (dev != l->device) return K3MOE_E_INVALID_ARG;
    const k3moe_config &c = l->cfg;
    const int64_t E = c.n_experts;
    const k3moe_mxfp4 *m[3] = {&l->w.gate, &l->w.up, &l->w.down};
    const CachePlan plan = cache_plan(c, n_slots);
    k3moe_cache tmp{};
    tmp.layer = l;
    tmp.S = n_slots;
    tmp.device = dev;
    for (int i = 0; i < 6; ++i) {
        const void *p = (i & 1) ? (const void *)m[i / 2]->scales : (const void *)m[i / 2]->packed;
        hipPointerAttribute_t a{};
        if (hipPointerGetAttributes(&a, p) != hipSuccess) {
            (void)hipGetLastError();
            return K3MOE_E_INVALID_ARG;  // pageable host memory: the device cannot read it
        }
        void *dp = nullptr;
        if (a.type == hipMemoryTypeHost) {  // pinned host pages: their address on the device
            if (hipHostGetDevicePointer(&dp, const_cast<void *>(p), 0) != hipSuccess) {
                (void)hipGetLastError();
                return K3MOE_E_INVALID_ARG;
            }
        } else if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
            dp = const_cast<void *>(p);
        }
        if (!dp || !aligned(dp, 16)) return K3MOE_E_INVALID_ARG;
        tmp.src[i] = static_cast<const uint8_t *>(dp);
        tmp.src_stride[i] = (i & 1) ? m[i / 2]->expert_stride_scales : m[i / 2]->expert_stride_packed;
        tmp.seg_len[i] = plan.seg_len[i];
        tmp.seg_off[i] = plan.seg_off[i];
    }
    tmp.slot_bytes = plan.slot_bytes;
    tmp.expert_bytes = plan.expert_bytes;
    const size_t table = plan.table;
    // everything the cache allocates is added up before anything is allocated
    size_t free_b = 0;
    const k3moe_status fs = free_hbm(&free_b);
    if (fs != K3MOE_OK) return fs;
    if (plan.arena + table + kCreateMarginBytes > free_b) return K3MOE_E_OUT_OF_MEMORY;
    k3moe_cache *cc = new (std::nothrow) k3moe_cache(tmp);
    if (!cc) return K3MOE_E_OUT_OF_MEMORY;
    if (hipMalloc(&cc->arena, (size_t)cc->slot_bytes * n_slots) != hipSuccess) {
        delete cc;
        return K3MOE_E_OUT_OF_MEMORY;
    }
    if (hipMalloc(&cc->table, table) != hipSuccess) {
        (void)hipFree(cc->arena);
        delete cc;
        return K3MOE_E_OUT_OF_MEMORY;
    }
    size_t o = 0;
    cc->ctr = reinterpret_cast<unsigned long long *>(cc->table + o);
    o += align256(sizeof(unsigned long long) * kCtrCount);
    cc->slot_of = reinterpret_cast<int32_t *>(cc->table + o);
    o += align256(sizeof(int32_t) * E);
    cc->key_of = reinterpret_cast<int32_t *>(cc->table + o);
    o += align256(sizeof(int32_t) * n_slots);
    cc->used_at = reinterpret_cast<long long *>(cc->table + o);
    if (launch_cache_init(cc->ctr, cc->slot_of, (int)E, cc->key_of, cc->used_at, n_slots, nullptr) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(cc->table);
        (void)hipFree(cc->arena);
        delete cc;
        return K3MOE_E_HIP;
    }
    *out = cc;
    return K3MOE_OK;
}

k3moe_status k3moe_cache_device_bytes(const k3moe_config *cfg, int32_t n_slots, size_t *bytes)
{
    if (!bytes) return K3MOE_E_INVALID_ARG;
    const k3moe_status s = check_config(cfg);
    if (s != K3MOE_OK) return s;
    if (n_slots < 1 || n_slots > cfg->n_experts) return K3MOE_E_INVALID_ARG;
    const CachePlan p = cache_plan(*cfg, n_slots);
    *bytes = p.arena + p.table;
    return K3MOE_OK;
}

k3moe_status k3moe_cache_workspace_size(const k3moe_cache *c, int32_t max_tokens, size_t *bytes)
{
    if (!c || !bytes || max_tokens < 0) return K3MOE_E_INVALID_ARG;
    if (!batch_fits(c->layer->cfg, max_tokens)) return K3MOE_E_UNSUPPORTED_SHAPE;
    // enough for the layer's own route/forward too, so one workspace serves a step
    *bytes = std::max(cache_ws(c, max_tokens).total, ws_layout(c->layer->cfg, max_tokens).total);
    return K3MOE_OK;
}

k3moe_status k3moe_cache_forward(k3moe_cache *c, const uint16_t *x, int32_t T, const int32_t *idx,
                                 const float *w, float *out, void *ws, size_t ws_bytes, void *stream)
{
    if (!c || T < 0) return K3MOE_E_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return K3MOE_E_HIP;
    if (dev != c->device) return K3MOE_E_INVALID_ARG;
    if (T == 0) return K3MOE_OK;
    const k3moe_config &cfg = c->layer->cfg;
    if (!batch_fits(cfg, T)) return K3MOE_E_UNSUPPORTED_SHAPE;
    if (!x || !idx || !w || !out) return K3MOE_E_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(out, 16)) return K3MOE_E_ALIGNMENT;
    const CacheWs cw = cache_ws(c, T);
    if (!ws || !aligned(ws, 256) || ws_bytes < cw.total) return K3MOE_E_WORKSPACE;
    char *wsc = static_cast<char *>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = (int64_t)T * cfg.topk;
    CachePlanParams pp{};
    pp.idx = idx;
    pp.n = n;
    pp.E = cfg.n_experts;
    pp.S = c->S;
    pp.expert_bytes = c->expert_bytes;
    pp.slot_of = c->slot_of;
    pp.key_of = c->key_of;
    pp.used_at = c->used_at;
    pp.ctr = c->ctr;
    pp.remap = reinterpret_cast<int32_t *>(wsc + cw.remap);
    pp.fill = reinterpret_cast<int2 *>(wsc + cw.fill);
    pp.nfill = reinterpret_cast<int32_t *>(wsc + cw.nfill);
    CacheFillParams fp{};
    fp.fill = pp.fill;
    fp.nfill = pp.nfill;
    for (int i = 0; i < 6; ++i) {
        fp.src[i] = c->src[i];
        fp.src_stride[i] = c->src_stride[i];
        fp.seg_len[i] = c->seg_len[i];
        fp.seg_off[i] = c->seg_off[i];
    }
    fp.arena = c->arena;
    fp.slot_bytes = c->slot_bytes;
    fp.expert_bytes = c->expert_bytes;
    fp.nchunk = (int)((c->expert_bytes + kFillChunk - 1) / kFillChunk);
    const int max_fill = (int)std::min<int64_t>(c->S, std::min<int64_t>(cfg.n_experts, n));
    if (launch_cache_plan_fill(pp, fp, max_fill, st, c->layer->prof) != hipSuccess) return K3MOE_E_HIP;
    if (launch_forward(cache_view(c), x, T, pp.remap, w, out, wsc, cw.lay, st, c->layer->prof) != hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_cache_stats_read(const k3moe_cache *c, k3moe_cache_stats *out, void *stream)
{
    if (!c || !out) return K3MOE_E_INVALID_ARG;
    unsigned long long v[kCtrCount];
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(v, c->ctr, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess) return K3MOE_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return K3MOE_E_HIP;
    out->steps = v[kCtrSteps];
    out->requests = v[kCtrRequests];
    out->resident_hits = v[kCtrHits];
    out->misses = v[kCtrMisses];
    out->evictions = v[kCtrEvictions];
    out->dropped = v[kCtrDropped];
    out->bytes_read = v[kCtrBytes];
    return K3MOE_OK;
}

k3moe_status k3moe_cache_slots(const k3moe_cache *c, int32_t *slots, void *stream)
{
    if (!c || !slots) return K3MOE_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(slots, c->key_of, sizeof(int32_t) * c->S, hipMemcpyDeviceToHost, st) != hipSuccess)
        return K3MOE_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return K3MOE_E_HIP;
    return K3MOE_OK;
}

k3moe_status k3moe_cache_reset(k3moe_cache *c, void *stream)
{
    if (!c) return K3MOE_E_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return K3MOE_E_HIP;
    if (dev != c->device) return K3MOE_E_INVALID_ARG;  // the table lives on the cache's device
    if (launch_cache_init(c->ctr, c->slot_of, c->layer->cfg.n_experts, c->key_of, c->used_at, c->S,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
        return K3MOE_E_HIP;
    return K3MOE_OK;
}

void k3moe_cache_destroy(k3moe_cache *c)
{
    if (!c) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(c->table);
    (void)hipFree(c->arena);
    delete c;
}

void k3moe_layer_destroy(k3moe_layer *l)
{
    if (!l) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(l->errors);
    for (const Profiler::Rec &r : l->prof->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : l->prof->spare) (void)hipEventDestroy(e);
    delete l->prof;
    delete l;
}

const char *k3moe_status_string(k3moe_status s)
{
    // a C caller may pass any int; read it as one (loading a C++ enum
    // outside its value range is undefined)
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case K3MOE_OK: return "ok";
    case K3MOE_E_INVALID_ARG: return "invalid argument";
    case K3MOE_E_CONFIG: return "invalid or incomplete config";
    case K3MOE_E_UNSUPPORTED_SHAPE: return "unsupported shape";
    case K3MOE_E_ALIGNMENT: return "pointer or stride not aligned";
    case K3MOE_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case K3MOE_E_OUT_OF_MEMORY: return "out of device memory";
    case K3MOE_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
