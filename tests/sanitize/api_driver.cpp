// Drives the C ABI's host-side validation (config and weight descriptors,
// argument checks, the cache planner, status strings) for a build of the
// library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
// (the kimi-k3-in-c README, Part I "Common questions", builds its C with
// both). Every call here returns before the first HIP runtime call, so it
// runs without a GPU. Prints "ok" and exits 0 when each status is the one
// the header documents.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "k3moe.h"

// The HIP runtime keeps process-lifetime allocations of its own; leak
// reports would be about those, so only memory errors and undefined
// behaviour are checked.
extern "C" const char *__asan_default_options() { return "detect_leaks=0"; }

static int failures = 0;

#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        const int got_ = (int)(call);                                                         \
        if (got_ != (int)(want)) {                                                            \
            std::fprintf(stderr, "%s:%d: %s gave %d, want %d\n", __FILE__, __LINE__, #call, got_, \
                         (int)(want));                                                        \
            failures++;                                                                       \
        }                                                                                     \
    } while (0)

static k3moe_config base_config()
{
    k3moe_config c;
    std::memset(&c, 0, sizeof c);
    c.struct_size = sizeof(k3moe_config);
    c.abi_version = K3MOE_ABI_VERSION;
    c.hidden = 7168;
    c.inter = 1536;
    c.n_experts = 896;
    c.topk = 16;
    c.shared_inter = 1536;
    c.renorm = 1;
    c.routed_scale = 1.0f;
    c.act = K3MOE_ACT_SITU;
    c.situ_b1 = 4.0f;
    c.situ_b2 = 25.0f;
    return c;
}

// Descriptors that pass validation: addresses are never dereferenced by
// the checks, only tested for alignment and presence.
static k3moe_weights base_weights(const k3moe_config &c)
{
    alignas(256) static unsigned char arena[4096];
    k3moe_weights w;
    std::memset(&w, 0, sizeof w);
    const int64_t ek = c.latent ? c.latent : c.hidden;
    w.router_w = reinterpret_cast<const uint16_t *>(arena);
    w.router_bias = reinterpret_cast<const float *>(arena + 256);
    k3moe_mxfp4 *m[3] = {&w.gate, &w.up, &w.down};
    for (int i = 0; i < 3; ++i) {
        m[i]->packed = arena + 512 + 512 * i;
        m[i]->scales = arena + 768 + 512 * i;
        m[i]->expert_stride_packed = (int64_t)c.inter * ek / 2;
        m[i]->expert_stride_scales = (int64_t)c.inter * ek / 32;
    }
    if (c.shared_inter) {
        w.sh_gate = reinterpret_cast<const uint16_t *>(arena + 2048);
        w.sh_up = reinterpret_cast<const uint16_t *>(arena + 2304);
        w.sh_down = reinterpret_cast<const uint16_t *>(arena + 2560);
    }
    if (c.latent) {
        w.lat_down = reinterpret_cast<const uint16_t *>(arena + 2816);
        w.lat_up = reinterpret_cast<const uint16_t *>(arena + 3072);
        if (c.latent_norm) w.lat_norm = reinterpret_cast<const float *>(arena + 3328);
    }
    return w;
}

static void config_refusals()
{
    k3moe_layer *l = reinterpret_cast<k3moe_layer *>(0x1);
    k3moe_config c = base_config();
    k3moe_weights w = base_weights(c);
    EXPECT(k3moe_layer_create(&c, &w, nullptr), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_layer_create(nullptr, &w, &l), K3MOE_E_INVALID_ARG);
    if (l != nullptr) failures++;   // *out is cleared on every refusal
    struct Case {
        void (*edit)(k3moe_config &);
        k3moe_status want;
    };
    const Case cases[] = {
        {[](k3moe_config &c) { c.struct_size -= 4; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.abi_version += 1; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.hidden = 0; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.inter = -128; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.topk = 897; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.renorm = 2; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.act = 0; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.routed_scale = NAN; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.situ_b2 = 0.0f; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.situ_b1 = INFINITY; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.hidden = 7100; }, K3MOE_E_UNSUPPORTED_SHAPE},
        {[](k3moe_config &c) { c.shared_inter = 100; }, K3MOE_E_UNSUPPORTED_SHAPE},
        {[](k3moe_config &c) { c.n_experts = 5000; c.topk = 16; }, K3MOE_E_UNSUPPORTED_SHAPE},
        {[](k3moe_config &c) { c.topk = 65; }, K3MOE_E_UNSUPPORTED_SHAPE},
        {[](k3moe_config &c) { c.latent = -128; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.latent_norm = 1; }, K3MOE_E_CONFIG},   // norm without a latent
        {[](k3moe_config &c) { c.latent = 3584; c.latent_norm = 1; c.rms_eps = 0.0f; }, K3MOE_E_CONFIG},
        {[](k3moe_config &c) { c.latent = 3500; }, K3MOE_E_UNSUPPORTED_SHAPE},
        {[](k3moe_config &c) { c.hidden = 65536; c.inter = 32768; }, K3MOE_E_UNSUPPORTED_SHAPE},
    };
    for (const Case &cs : cases) {
        k3moe_config b = base_config();
        cs.edit(b);
        l = reinterpret_cast<k3moe_layer *>(0x1);
        EXPECT(k3moe_layer_create(&b, &w, &l), cs.want);
        if (l != nullptr) failures++;
    }
}

static void weight_refusals()
{
    const k3moe_config c = base_config();
    k3moe_layer *l = nullptr;
    EXPECT(k3moe_layer_create(&c, nullptr, &l), K3MOE_E_INVALID_ARG);
    {
        k3moe_weights w = base_weights(c);
        w.router_w = nullptr;
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_weights w = base_weights(c);
        w.router_w = reinterpret_cast<const uint16_t *>(reinterpret_cast<uintptr_t>(w.router_w) + 2);
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_ALIGNMENT);
    }
    {
        k3moe_weights w = base_weights(c);
        w.gate.expert_stride_packed -= 16;   // experts would overlap
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_weights w = base_weights(c);
        w.down.expert_stride_scales += 8;    // not a multiple of 16
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_ALIGNMENT);
    }
    {
        k3moe_weights w = base_weights(c);
        w.up.scales = nullptr;
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_weights w = base_weights(c);
        w.sh_down = nullptr;                 // a shared expert needs all three
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_config c0 = base_config();
        c0.shared_inter = 0;
        k3moe_weights w = base_weights(c);   // shared pointers given, none configured
        EXPECT(k3moe_layer_create(&c0, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_weights w = base_weights(c);
        w.lat_down = w.router_w;             // latent pointers on a flat layer
        EXPECT(k3moe_layer_create(&c, &w, &l), K3MOE_E_INVALID_ARG);
    }
    {
        k3moe_config cl = base_config();
        cl.latent = 3584;
        cl.latent_norm = 1;
        cl.rms_eps = 1e-5f;
        k3moe_weights w = base_weights(cl);
        w.lat_norm = nullptr;                // the norm's gain is required
        EXPECT(k3moe_layer_create(&cl, &w, &l), K3MOE_E_INVALID_ARG);
        w = base_weights(cl);
        w.lat_up = reinterpret_cast<const uint16_t *>(reinterpret_cast<uintptr_t>(w.lat_up) + 4);
        EXPECT(k3moe_layer_create(&cl, &w, &l), K3MOE_E_ALIGNMENT);
    }
}

static void call_refusals()
{
    size_t n = 0;
    uint64_t cnt = 0;
    EXPECT(k3moe_workspace_size(nullptr, 1, &n), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_route(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_forward(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_route_forward(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_forward_residual(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_step(nullptr, nullptr, 1, nullptr, 1e-5f, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_forward_noalloc(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_error_count(nullptr, &cnt, nullptr), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_profile_enable(nullptr, 1), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_cache_create(nullptr, 4, nullptr), K3MOE_E_INVALID_ARG);
    k3moe_cache *cc = reinterpret_cast<k3moe_cache *>(0x1);
    EXPECT(k3moe_cache_create(nullptr, 4, &cc), K3MOE_E_INVALID_ARG);
    if (cc != nullptr) failures++;
    EXPECT(k3moe_cache_workspace_size(nullptr, 1, &n), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_cache_forward(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           K3MOE_E_INVALID_ARG);
    k3moe_layer_destroy(nullptr);
    k3moe_cache_destroy(nullptr);
}

static void cache_planner()
{
    k3moe_config c = base_config();
    size_t n = 0;
    const size_t slot = 3 * (1536 * 7168 / 2 + 1536 * 7168 / 32);
    EXPECT(k3moe_cache_device_bytes(&c, 224, &n), K3MOE_OK);
    if (!(n > 224 * slot && n < 224 * slot + 65536)) failures++;
    EXPECT(k3moe_cache_device_bytes(&c, 0, &n), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_cache_device_bytes(&c, 897, &n), K3MOE_E_INVALID_ARG);
    EXPECT(k3moe_cache_device_bytes(&c, 1, nullptr), K3MOE_E_INVALID_ARG);
    c.latent = 3584;
    c.latent_norm = 1;
    c.rms_eps = 1e-5f;
    EXPECT(k3moe_cache_device_bytes(&c, 896, &n), K3MOE_OK);
    c.abi_version = 0;
    EXPECT(k3moe_cache_device_bytes(&c, 1, &n), K3MOE_E_CONFIG);
}

int main()
{
    for (int s = -2; s <= 9; ++s) {
        const char *m = k3moe_status_string(static_cast<k3moe_status>(s));
        if (!m || !*m) failures++;
    }
    config_refusals();
    weight_refusals();
    call_refusals();
    cache_planner();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
