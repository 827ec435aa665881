/*
 * Drives every entry of the oracle (oracle/k3moe_oracle.c) on small inputs
 * whose buffers are allocated at their exact sizes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (the kimi-k3-in-c README,
 * Part I "Common questions", builds its C with both). Shapes cover odd
 * widths and partial 32-groups, E8M0 bytes 0 and 255, ids out of range,
 * missing slots, no shared expert, the latent layer with and without its
 * norm, and the size refusals. Prints "ok" and exits 0 when every call
 * returns what its contract says.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

/* the oracle's entry points (compiled into this program) */
double k3o_e2m1(int code);
double k3o_e8m0(int b);
double k3o_bf16(uint16_t h);
void k3o_mxfp4_gemv(double *y, double *yabs, const double *x, const uint8_t *packed, const uint8_t *scales,
                    int64_t K, int64_t rows);
void k3o_bf16_gemv(double *y, double *yabs, const double *x, const uint16_t *W, int64_t K, int64_t rows);
double k3o_act(double g, double u, int kind, double b1, double b2);
int k3o_route(int32_t *idx, float *w, double *logits_out, float *ch_out, const uint16_t *x, const uint16_t *Wr,
              const float *bias, int64_t T, int64_t H, int64_t E, int64_t topk, int renorm, float routed_scale);
int64_t k3o_forward(double *out, double *denom, const uint16_t *x, int64_t T, int64_t H, int64_t I,
                    const int32_t *idx, const float *w, int64_t topk, int64_t E, const int32_t *slot_of,
                    const uint8_t *gate_packed, const uint8_t *gate_scales, const uint8_t *up_packed,
                    const uint8_t *up_scales, const uint8_t *down_packed, const uint8_t *down_scales,
                    const uint16_t *sh_gate, const uint16_t *sh_up, const uint16_t *sh_down, int64_t Is, int act,
                    double b1, double b2);
double k3o_rmsnorm(double *out, const double *v, const float *gamma, int64_t n, double eps);
int64_t k3o_forward_latent(double *out, double *denom, const uint16_t *x, int64_t T, int64_t H, int64_t L,
                           int64_t I, const int32_t *idx, const float *w, int64_t topk, int64_t E,
                           const int32_t *slot_of, const uint8_t *gate_packed, const uint8_t *gate_scales,
                           const uint8_t *up_packed, const uint8_t *up_scales, const uint8_t *down_packed,
                           const uint8_t *down_scales, const uint16_t *lat_down, const uint16_t *lat_up, int norm,
                           const float *gamma, double eps, const uint16_t *sh_gate, const uint16_t *sh_up,
                           const uint16_t *sh_down, int64_t Is, int act, double b1, double b2);
int k3o_threads(void);
uint16_t k3o_bf16_rne(float v);
void k3o_prenorm_bf16(uint16_t *x, const float *h, const float *gamma, int64_t T, int64_t n, float eps);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint64_t next(void)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* n bytes of random nibbles; scale bytes near 127 with some 0 and 255 */
static uint8_t *rand_bytes(size_t n)
{
    uint8_t *p = xmalloc(n);
    for (size_t i = 0; i < n; i++) p[i] = (uint8_t)next();
    return p;
}

static uint8_t *rand_scales(size_t n)
{
    uint8_t *p = xmalloc(n);
    for (size_t i = 0; i < n; i++) {
        const uint64_t r = next() % 16;
        p[i] = r == 0 ? 255 : r == 1 ? 0 : (uint8_t)(120 + r);
    }
    return p;
}

/* bf16 patterns of values in about [-1, 1] */
static uint16_t *rand_bf16(size_t n)
{
    uint16_t *p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; i++) {
        const float f = (float)((double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0);
        p[i] = k3o_bf16_rne(f);
    }
    return p;
}

static int failures = 0;

#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            failures++;                                             \
        }                                                           \
    } while (0)

static int all_finite(const double *v, size_t n)
{
    for (size_t i = 0; i < n; i++)
        if (!isfinite(v[i])) return 0;
    return 1;
}

static void gemv_cases(void)
{
    const int64_t Ks[] = {1, 7, 32, 33, 64, 100};
    for (size_t c = 0; c < sizeof Ks / sizeof Ks[0]; c++) {
        const int64_t K = Ks[c], rows = 3;
        const int64_t rb = (K + 1) / 2, ng = (K + 31) / 32;
        uint8_t *p = rand_bytes((size_t)(rows * rb)), *s = rand_scales((size_t)(rows * ng));
        double *x = xmalloc(sizeof(double) * (size_t)K), *y = xmalloc(sizeof(double) * rows),
               *ya = xmalloc(sizeof(double) * rows);
        for (int64_t i = 0; i < K; i++) x[i] = (double)(i % 5) - 2.0;
        k3o_mxfp4_gemv(y, ya, x, p, s, K, rows);
        for (int64_t o = 0; o < rows; o++) CHECK(isfinite(y[o]) && ya[o] >= fabs(y[o]));
        k3o_mxfp4_gemv(y, NULL, x, p, s, K, rows);
        uint16_t *W = rand_bf16((size_t)(rows * K));
        k3o_bf16_gemv(y, ya, x, W, K, rows);
        for (int64_t o = 0; o < rows; o++) CHECK(isfinite(y[o]) && ya[o] >= fabs(y[o]));
        free(p); free(s); free(x); free(y); free(ya); free(W);
    }
    for (int code = 0; code < 16; code++) CHECK(fabs(k3o_e2m1(code)) <= 6.0);
    CHECK(k3o_e8m0(255) == 0.0 && k3o_e8m0(127) == 1.0 && k3o_e8m0(0) > 0.0);
}

static void route_cases(void)
{
    const int64_t T = 3, H = 96, E = 5;
    uint16_t *x = rand_bf16((size_t)(T * H)), *Wr = rand_bf16((size_t)(E * H));
    float *bias = xmalloc(sizeof(float) * E);
    for (int64_t e = 0; e < E; e++) bias[e] = (float)e * 0.01f;
    for (int64_t k = 1; k <= E; k += E - 1) {
        int32_t *idx = xmalloc(sizeof(int32_t) * (size_t)(T * k));
        float *w = xmalloc(sizeof(float) * (size_t)(T * k));
        double *lg = xmalloc(sizeof(double) * (size_t)(T * E));
        float *ch = xmalloc(sizeof(float) * (size_t)(T * E));
        for (int renorm = 0; renorm < 2; renorm++) {
            CHECK(k3o_route(idx, w, lg, ch, x, Wr, renorm ? bias : NULL, T, H, E, k, renorm, 2.5f) == 0);
            for (int64_t i = 0; i < T * k; i++) CHECK(idx[i] >= 0 && idx[i] < E && w[i] >= 0.0f);
            CHECK(k3o_route(idx, w, NULL, NULL, x, Wr, bias, T, H, E, k, renorm, 1.0f) == 0);
        }
        CHECK(k3o_route(idx, w, NULL, NULL, x, Wr, bias, 0, H, E, k, 1, 1.0f) == 0);   /* T = 0 */
        free(idx); free(w); free(lg); free(ch);
    }
    int32_t idx1[8];
    float w1[8];
    CHECK(k3o_route(idx1, w1, NULL, NULL, x, Wr, bias, T, H, E, E + 1, 1, 1.0f) == -1);  /* topk > E */
    CHECK(k3o_route(idx1, w1, NULL, NULL, x, Wr, bias, -1, H, E, 1, 1, 1.0f) == -1);
    free(x); free(Wr); free(bias);
}

struct experts {
    uint8_t *gp, *gs, *up, *us, *dp, *ds;
};

static struct experts make_experts(int64_t n, int64_t I, int64_t K)
{
    struct experts x;
    x.gp = rand_bytes((size_t)(n * I * K / 2));
    x.gs = rand_scales((size_t)(n * I * K / 32));
    x.up = rand_bytes((size_t)(n * I * K / 2));
    x.us = rand_scales((size_t)(n * I * K / 32));
    x.dp = rand_bytes((size_t)(n * K * I / 2));
    x.ds = rand_scales((size_t)(n * K * I / 32));
    return x;
}

static void free_experts(struct experts *x)
{
    free(x->gp); free(x->gs); free(x->up); free(x->us); free(x->dp); free(x->ds);
}

static void forward_cases(void)
{
    const int64_t T = 2, H = 64, I = 32, K = 3, E = 6, Is = 32, nslot = 4;
    uint16_t *x = rand_bf16((size_t)(T * H));
    struct experts ex = make_experts(nslot, I, H);
    int32_t slot_of[6] = {0, -1, 1, 2, -1, 3};
    /* token 0: experts 0, 2 and an id past the end; token 1: 5, -1, 3 */
    int32_t idx[6] = {0, 2, 6, 5, -1, 3};
    float w[6] = {0.5f, 0.25f, 0.25f, 0.6f, 0.3f, 0.1f};
    uint16_t *s1 = rand_bf16((size_t)(Is * H)), *s3 = rand_bf16((size_t)(Is * H)), *s2 = rand_bf16((size_t)(H * Is));
    double *out = xmalloc(sizeof(double) * (size_t)(T * H)), *den = xmalloc(sizeof(double) * (size_t)(T * H));
    for (int act = 1; act <= 2; act++) {
        CHECK(k3o_forward(out, den, x, T, H, I, idx, w, K, E, slot_of, ex.gp, ex.gs, ex.up, ex.us, ex.dp, ex.ds,
                          s1, s3, s2, Is, act, 4.0, 25.0) == 2);
        CHECK(all_finite(out, (size_t)(T * H)) && all_finite(den, (size_t)(T * H)));
        CHECK(k3o_forward(out, NULL, x, T, H, I, idx, w, K, E, slot_of, ex.gp, ex.gs, ex.up, ex.us, ex.dp, ex.ds,
                          NULL, NULL, NULL, 0, act, 4.0, 25.0) == 2);
    }
    int32_t missing[6] = {1, 0, 2, 3, 5, 0};   /* expert 1 has no slot */
    CHECK(k3o_forward(out, den, x, T, H, I, missing, w, K, E, slot_of, ex.gp, ex.gs, ex.up, ex.us, ex.dp, ex.ds,
                      s1, s3, s2, Is, 1, 4.0, 25.0) == -1);
    CHECK(k3o_forward(out, den, x, T, H, I, idx, w, K, E, slot_of, ex.gp, ex.gs, ex.up, ex.us, ex.dp, ex.ds,
                      s1, s3, s2, Is, 3, 4.0, 25.0) == -1);   /* no such activation */

    /* latent: width L = 32 between the projections */
    const int64_t L = 32;
    struct experts lx = make_experts(nslot, I, L);
    uint16_t *wd = rand_bf16((size_t)(L * H)), *wu = rand_bf16((size_t)(H * L));
    float *gamma = xmalloc(sizeof(float) * L);
    for (int64_t l = 0; l < L; l++) gamma[l] = 1.0f + 0.01f * (float)l;
    for (int norm = 0; norm < 2; norm++) {
        CHECK(k3o_forward_latent(out, den, x, T, H, L, I, idx, w, K, E, slot_of, lx.gp, lx.gs, lx.up, lx.us, lx.dp,
                                 lx.ds, wd, wu, norm, norm ? gamma : NULL, 1e-5, s1, s3, s2, Is, 1, 4.0,
                                 25.0) == 2);
        CHECK(all_finite(out, (size_t)(T * H)) && all_finite(den, (size_t)(T * H)));
    }
    CHECK(k3o_forward_latent(out, den, x, T, H, 0, I, idx, w, K, E, slot_of, lx.gp, lx.gs, lx.up, lx.us, lx.dp,
                             lx.ds, wd, wu, 1, gamma, 1e-5, s1, s3, s2, Is, 1, 4.0, 25.0) == -1);
    free_experts(&lx); free(wd); free(wu); free(gamma);
    free_experts(&ex); free(x); free(s1); free(s3); free(s2); free(out); free(den);
}

static void norm_cases(void)
{
    const int64_t T = 2, n = 96;
    float *h = xmalloc(sizeof(float) * (size_t)(T * n)), *g = xmalloc(sizeof(float) * n);
    for (int64_t i = 0; i < T * n; i++) h[i] = (float)((int64_t)(next() % 2001) - 1000) * 0.01f;
    for (int64_t i = 0; i < n; i++) g[i] = 1.0f;
    uint16_t *xo = xmalloc(sizeof(uint16_t) * (size_t)(T * n));
    k3o_prenorm_bf16(xo, h, g, T, n, 1e-5f);
    double *v = xmalloc(sizeof(double) * n), *o = xmalloc(sizeof(double) * n);
    for (int64_t i = 0; i < n; i++) v[i] = h[i];
    const double inv = k3o_rmsnorm(o, v, g, n, 1e-5);
    CHECK(isfinite(inv) && inv > 0.0);
    CHECK(k3o_rmsnorm(v, v, NULL, n, 1e-5) > 0.0);   /* in place, no gain */
    CHECK(k3o_act(0.0, 3.0, 1, 4.0, 25.0) == 0.0);
    CHECK(k3o_threads() >= 1);
    free(h); free(g); free(xo); free(v); free(o);
}

int main(void)
{
    gemv_cases();
    route_cases();
    forward_cases();
    norm_cases();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
