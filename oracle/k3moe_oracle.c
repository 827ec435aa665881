/*
 * k3moe oracle: a plain, slow, fp64 CPU statement of the sigmoid-routed MXFP4
 * expert layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product path (libk3moe.so and its
 * Python binding) never links, loads or calls it, and shares no code with it.
 *
 * What is computed, and where it is stated (page: "kimi-k3-in-c" README,
 * FareedKhan-dev, as captured on brainstate.renovationsteps.com):
 *   - MXFP4 format: §4 "Reduction one: the experts already ship at half a
 *     byte" (the E2M1 value table, the E8M0 exponent byte, one scale per 32
 *     weights, the low nibble holding the even-indexed weight, scale byte 255
 *     treated as zero so the group drops out, and the matrix-vector product
 *     that multiplies straight from the nibbles with a double accumulator per
 *     32-group scaled once per group).
 *   - bf16 widening: §5 "Kernels with a floating point contract" (a bf16 is
 *     the top half of an fp32, so widening is exact).
 *   - Router: §9 "Picking 16 experts of 896", k3_router (sigmoid score, bias
 *     added for selection only, top-k by repeated maximum with the lowest index
 *     winning ties, weights from the unbiased score, optional renormalisation,
 *     then the routed scale).
 *   - Layer: §9, k3_moe steps 3 and 6 and k3_situ_glu (each selected expert:
 *     gate and up projections, SiTU-GLU, down projection; weighted sum in
 *     router order; the shared expert on the original input, added unweighted
 *     after the routed sum).
 *   - Latent layer: §9, all six steps of k3_moe (down-projection of x into
 *     the expert latent, the experts at the latent width, RMSNorm of the
 *     aggregate, up-projection, shared experts on the original x) and §5,
 *     k3_rmsnorm (epsilon inside the square root).
 *   - Pre-MoE norm of a decoder layer: the decoder-layer listing after
 *     "Aggregate, attend, aggregate again" (the MoE reads k3_rmsnorm of the
 *     residual stream with the post-attention gain) in the exact float form
 *     of §5 k3_rmsnorm, rounded once to the layer's bf16 tokens.
 * Expert failures that the pages count as drops are mirrored: an index outside
 * [0, n_experts) contributes nothing and is counted.
 *
 * Precision: everything is fp64 except where the pages fix fp32: the router's
 * score, selection score and weights are fp32 values (sc, ch, w), because the
 * selection is a decision taken in fp32 on the pages. The score is the fp32
 * value of the sigmoid of the fp32 logit, evaluated in fp64 and rounded once.
 *
 * The SwiGLU activation (g * sigmoid(g) * u) is a second activation kind the
 * layer can be configured with; the pages use SiTU-GLU. SwiGLU is pinned by
 * closed forms (the sigmoid is exactly 3/4 and 1/4 at +-ln 3, zero gate or
 * up, the large-gate limits) and by the SiTU limit of large betas.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define K3O_ACT_SITU 1
#define K3O_ACT_SWIGLU 2

/* E2M1 code -> value. Bit 3 is the sign; the 3 low bits index the eight
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (§4, the 16-entry table). Code 8 is
 * -0. Written out as the 16 signed values so the decode has no branch on the
 * (random) sign bit. */
static const double e2m1_value[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double k3o_e2m1(int code) { return e2m1_value[code & 15]; }

/* E8M0 byte -> 2^(b - 127); byte 255 (NaN in the MX specification) maps to 0
 * so its whole 32-group contributes nothing (§4). Byte 0 is 2^-127. */
double k3o_e8m0(int b)
{
    if (b == 255) return 0.0;
    return ldexp(1.0, b - 127);
}

/* bf16 bit pattern -> value: the pattern is the upper 16 bits of an fp32 (§5). */
double k3o_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The E2M1 code of column c in a packed row: byte c/2, low nibble when c is
 * even, high nibble when c is odd (§4, nibble order). */
static int nibble_at(const uint8_t *row, int64_t c)
{
    const uint8_t b = row[c / 2];
    return (c & 1) ? (b >> 4) : (b & 0x0F);
}

/* y[o] = sum_c W[o][c] * x[c] with W in MXFP4, rows x K (§4, the matrix-vector
 * product over packed nibbles). Row o has (K+1)/2 packed bytes and ceil(K/32)
 * scale bytes. Per 32-group: a plain fp64 dot over the group's codes, skipped
 * when the scale byte is 255, then scaled by the group's power of two and
 * added to the row's fp64 accumulator. yabs (optional) receives the same sum
 * over |W[o][c] * x[c]|, the magnitude the error metric divides by. */
void k3o_mxfp4_gemv(double *y, double *yabs, const double *x,
                    const uint8_t *packed, const uint8_t *scales,
                    int64_t K, int64_t rows)
{
    const int64_t ngroup = (K + 31) / 32;
    const int64_t rowbytes = (K + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < rows; o++) {
        const uint8_t *prow = packed + o * rowbytes;
        const uint8_t *srow = scales + o * ngroup;
        double acc = 0.0, accabs = 0.0;
        for (int64_t g = 0; g < ngroup; g++) {
            const double s = k3o_e8m0(srow[g]);
            if (s == 0.0) continue;
            const int64_t c0 = g * 32;
            const int64_t n = (c0 + 32 <= K) ? 32 : (K - c0);
            double part = 0.0, partabs = 0.0;
            for (int64_t k = 0; k < n; k++) {
                const double p = x[c0 + k] * k3o_e2m1(nibble_at(prow, c0 + k));
                part += p;
                partabs += fabs(p);
            }
            acc += part * s;
            accabs += partabs * s;
        }
        y[o] = acc;
        if (yabs) yabs[o] = accabs;
    }
}

/* y[o] = sum_c W[o][c] * x[c] with W in bf16, rows x K, fp64 accumulation. */
void k3o_bf16_gemv(double *y, double *yabs, const double *x, const uint16_t *W,
                   int64_t K, int64_t rows)
{
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < rows; o++) {
        const uint16_t *row = W + o * K;
        double acc = 0.0, accabs = 0.0;
        for (int64_t c = 0; c < K; c++) {
            const double p = k3o_bf16(row[c]) * x[c];
            acc += p;
            accabs += fabs(p);
        }
        y[o] = acc;
        if (yabs) yabs[o] = accabs;
    }
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Gated activation of one (gate, up) pair (§9, k3_situ_glu).
 * SiTU-GLU: b1*tanh(g/b1) * sigmoid(g) * b2*tanh(u/b2); the sigmoid reads the
 * raw gate g, not the capped one, and |result| <= b1*b2.
 * SwiGLU:   g * sigmoid(g) * u. */
double k3o_act(double g, double u, int kind, double b1, double b2)
{
    if (kind == K3O_ACT_SITU)
        return (b1 * tanh(g / b1) * sigmoid(g)) * (b2 * tanh(u / b2));
    if (kind == K3O_ACT_SWIGLU)
        return g * sigmoid(g) * u;
    return NAN;
}

/* One expert's selection score, and the order the router takes experts in:
 * the larger score first, equal scores by the lower expert index. */
struct choice {
    float ch;
    int32_t e;
};

static int by_choice(const void *pa, const void *pb)
{
    const struct choice *a = (const struct choice *)pa, *b = (const struct choice *)pb;
    if (a->ch > b->ch) return -1;
    if (a->ch < b->ch) return 1;
    return (a->e > b->e) - (a->e < b->e);
}

/* Router for T tokens (§9, k3_router).
 *   logit[e] = sum_i x[i] * Wr[e][i]            fp64 over exact bf16 products
 *   sc[e]    = fp32 of sigmoid(fp32 logit)      unbiased score
 *   ch[e]    = sc[e] + bias[e]  (fp32 add)      selection score
 *   selection: the experts ordered by ch, larger first, and among equal ch
 *     the lower expert index first (the order in which a repeated strict
 *     maximum takes them); the first topk of that order, in order
 *   w[j] = sc[idx[j]]; if renorm: s = sum_j w[j] (fp32, j order) and, if
 *   s > 0, w[j] /= s; finally w[j] *= routed_scale.
 * Outputs idx [T][topk], w [T][topk]; optional logits [T][E] (fp64) and
 * ch [T][E] (fp32) for margin checks. Returns 0, or -1 on bad sizes. */
int k3o_route(int32_t *idx, float *w, double *logits_out, float *ch_out,
              const uint16_t *x, const uint16_t *Wr, const float *bias,
              int64_t T, int64_t H, int64_t E, int64_t topk,
              int renorm, float routed_scale)
{
    if (T < 0 || H <= 0 || E <= 0 || topk <= 0 || topk > E) return -1;
    double *xd = (double *)malloc(sizeof(double) * H);
    double *logit = (double *)malloc(sizeof(double) * E);
    float *sc = (float *)malloc(sizeof(float) * E);
    float *ch = (float *)malloc(sizeof(float) * E);
    struct choice *order = (struct choice *)malloc(sizeof(struct choice) * E);
    if (!xd || !logit || !sc || !ch || !order) {
        free(xd); free(logit); free(sc); free(ch); free(order);
        return -1;
    }
    for (int64_t t = 0; t < T; t++) {
        for (int64_t i = 0; i < H; i++) xd[i] = k3o_bf16(x[t * H + i]);
        k3o_bf16_gemv(logit, NULL, xd, Wr, H, E);
        for (int64_t e = 0; e < E; e++) {
            const float l32 = (float)logit[e];
            sc[e] = (float)sigmoid((double)l32);
            ch[e] = sc[e] + (bias ? bias[e] : 0.0f);
        }
        for (int64_t e = 0; e < E; e++) { order[e].ch = ch[e]; order[e].e = (int32_t)e; }
        qsort(order, (size_t)E, sizeof *order, by_choice);
        int32_t *it = idx + t * topk;
        float *wt = w + t * topk;
        for (int64_t j = 0; j < topk; j++) {
            it[j] = order[j].e;
            wt[j] = sc[order[j].e];
        }
        if (renorm) {
            float s = 0.0f;
            for (int64_t j = 0; j < topk; j++) s += wt[j];
            if (s > 0.0f)
                for (int64_t j = 0; j < topk; j++) wt[j] /= s;
        }
        for (int64_t j = 0; j < topk; j++) wt[j] *= routed_scale;
        if (logits_out) memcpy(logits_out + t * E, logit, sizeof(double) * E);
        if (ch_out) memcpy(ch_out + t * E, ch, sizeof(float) * E);
    }
    free(xd); free(logit); free(sc); free(ch); free(order);
    return 0;
}

/* Expert layer for T tokens given their routes (§9, k3_moe steps 3 and 6).
 * For each token t:
 *   out = 0
 *   for j in router order: e = idx[t][j]
 *       e outside [0, E): counted as a drop, contributes nothing
 *       g = W1_e x, u = W3_e x (MXFP4), a = act(g, u), y = W2_e a (MXFP4)
 *       out += w[t][j] * y
 *   if a shared expert is present: out += S2 act(S1 x, S3 x) (bf16, unweighted)
 * denom (optional) receives, per output element, the magnitude sum
 *   sum_j |w_j| * sum_n |W2_e[o][n] a_j[n]|  +  sum_n |S2[o][n] a_s[n]|.
 * Expert weights are passed for a subset of experts ("slots"): slot_of[e] is
 * the slot holding expert e, or -1. Layouts: gate/up packed [slot][I][H/2],
 * scales [slot][I][H/32]; down packed [slot][H][I/2], scales [slot][H][I/32];
 * shared gate/up bf16 [Is][H], shared down bf16 [H][Is] (NULL when Is == 0).
 * Returns the number of dropped assignments, or -1 when a selected expert has
 * no slot or the sizes are invalid. */
int64_t k3o_forward(double *out, double *denom,
                    const uint16_t *x, int64_t T, int64_t H, int64_t I,
                    const int32_t *idx, const float *w, int64_t topk, int64_t E,
                    const int32_t *slot_of,
                    const uint8_t *gate_packed, const uint8_t *gate_scales,
                    const uint8_t *up_packed, const uint8_t *up_scales,
                    const uint8_t *down_packed, const uint8_t *down_scales,
                    const uint16_t *sh_gate, const uint16_t *sh_up,
                    const uint16_t *sh_down, int64_t Is,
                    int act, double b1, double b2)
{
    if (T < 0 || H <= 0 || I <= 0 || topk <= 0 || E <= 0 || Is < 0) return -1;
    if (act != K3O_ACT_SITU && act != K3O_ACT_SWIGLU) return -1;
    const int64_t gp = I * ((H + 1) / 2), gs = I * ((H + 31) / 32);
    const int64_t dp = H * ((I + 1) / 2), ds = H * ((I + 31) / 32);
    const int64_t inner = (I > Is) ? I : Is;
    double *xd = (double *)malloc(sizeof(double) * H);
    double *g = (double *)malloc(sizeof(double) * inner);
    double *u = (double *)malloc(sizeof(double) * inner);
    double *a = (double *)malloc(sizeof(double) * inner);
    double *y = (double *)malloc(sizeof(double) * H);
    double *yabs = (double *)malloc(sizeof(double) * H);
    int64_t drops = 0;
    if (!xd || !g || !u || !a || !y || !yabs) { drops = -1; goto done; }

    for (int64_t t = 0; t < T; t++) {
        double *ot = out + t * H;
        double *dt = denom ? denom + t * H : NULL;
        for (int64_t i = 0; i < H; i++) xd[i] = k3o_bf16(x[t * H + i]);
        for (int64_t o = 0; o < H; o++) { ot[o] = 0.0; if (dt) dt[o] = 0.0; }

        for (int64_t j = 0; j < topk; j++) {
            const int32_t e = idx[t * topk + j];
            if (e < 0 || e >= E) { drops++; continue; }
            const int32_t s = slot_of[e];
            if (s < 0) { drops = -1; goto done; }
            k3o_mxfp4_gemv(g, NULL, xd, gate_packed + s * gp, gate_scales + s * gs, H, I);
            k3o_mxfp4_gemv(u, NULL, xd, up_packed + s * gp, up_scales + s * gs, H, I);
            for (int64_t n = 0; n < I; n++) a[n] = k3o_act(g[n], u[n], act, b1, b2);
            k3o_mxfp4_gemv(y, yabs, a, down_packed + s * dp, down_scales + s * ds, I, H);
            const double wj = (double)w[t * topk + j];
            for (int64_t o = 0; o < H; o++) {
                ot[o] += wj * y[o];
                if (dt) dt[o] += fabs(wj) * yabs[o];
            }
        }
        if (Is > 0) {
            k3o_bf16_gemv(g, NULL, xd, sh_gate, H, Is);
            k3o_bf16_gemv(u, NULL, xd, sh_up, H, Is);
            for (int64_t n = 0; n < Is; n++) a[n] = k3o_act(g[n], u[n], act, b1, b2);
            k3o_bf16_gemv(y, yabs, a, sh_down, Is, H);
            for (int64_t o = 0; o < H; o++) {
                ot[o] += y[o];
                if (dt) dt[o] += yabs[o];
            }
        }
    }
done:
    free(xd); free(g); free(u); free(a); free(y); free(yabs);
    return drops;
}

/* RMSNorm of n values (§5 "Kernels with a floating point contract",
 * k3_rmsnorm): inv = 1 / sqrt(sum_i v_i^2 / n + eps), epsilon inside the
 * square root; out_i = v_i * inv * gamma_i (gamma NULL: 1). fp64 throughout.
 * Returns inv. out may equal v. */
double k3o_rmsnorm(double *out, const double *v, const float *gamma, int64_t n, double eps)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += v[i] * v[i];
    const double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++) out[i] = v[i] * inv * (gamma ? (double)gamma[i] : 1.0);
    return inv;
}

/* Stable LatentMoE layer for T tokens (§9 "Picking 16 experts of 896", the
 * six steps of k3_moe): the experts run in a narrow latent of width L.
 *   z    = Wd x                           down-projection (bf16 [L][H])
 *   accL = sum_j w_j * W2_e act(W1_e z, W3_e z)   experts at width L (gate/up
 *          [I][L], down [L][I]), router order; bad ids counted, skipped
 *   accN = RMSNorm(accL) with gamma, if norm  (the AGGREGATE is normed, not
 *          each expert); else accN = accL
 *   out  = Wu accN                        up-projection (bf16 [H][L])
 *   out += S2 act(S1 x, S3 x)             shared expert on the ORIGINAL x,
 *                                         unweighted, after the routed part
 * The routing (idx, w) comes from k3o_route on the full-width x.
 * denom (optional), per output element o: the magnitude the output is made
 * of, propagated through each step,
 *   DL[l] = sum_j |w_j| sum_n |W2_e[l][n] a_j[n]|        (routed sum)
 *   DN[l] = inv |gamma_l| DL[l] + |accN[l]| * (sum_m |accL[m]| DL[m]) / ss
 *           (the second term: the norm's own dependence on every accL[m];
 *           without the norm DN = DL)
 *   denom[o] = sum_l |Wu[o][l]| DN[l] + sum_n |S2[o][n] a_s[n]|.
 * Returns the number of dropped assignments, or -1 (missing slot, sizes). */
int64_t k3o_forward_latent(double *out, double *denom,
                           const uint16_t *x, int64_t T, int64_t H, int64_t L, int64_t I,
                           const int32_t *idx, const float *w, int64_t topk, int64_t E,
                           const int32_t *slot_of,
                           const uint8_t *gate_packed, const uint8_t *gate_scales,
                           const uint8_t *up_packed, const uint8_t *up_scales,
                           const uint8_t *down_packed, const uint8_t *down_scales,
                           const uint16_t *lat_down, const uint16_t *lat_up,
                           int norm, const float *gamma, double eps,
                           const uint16_t *sh_gate, const uint16_t *sh_up,
                           const uint16_t *sh_down, int64_t Is,
                           int act, double b1, double b2)
{
    if (T < 0 || H <= 0 || L <= 0 || I <= 0 || topk <= 0 || E <= 0 || Is < 0) return -1;
    if (act != K3O_ACT_SITU && act != K3O_ACT_SWIGLU) return -1;
    if (!lat_down || !lat_up) return -1;
    const int64_t gp = I * ((L + 1) / 2), gs = I * ((L + 31) / 32);
    const int64_t dp = L * ((I + 1) / 2), ds = L * ((I + 31) / 32);
    int64_t inner = (I > Is) ? I : Is;
    if (L > inner) inner = L;
    const int64_t wide = (H > inner) ? H : inner;
    double *xd = (double *)malloc(sizeof(double) * H);
    double *z = (double *)malloc(sizeof(double) * L);
    double *g = (double *)malloc(sizeof(double) * inner);
    double *u = (double *)malloc(sizeof(double) * inner);
    double *a = (double *)malloc(sizeof(double) * inner);
    double *y = (double *)malloc(sizeof(double) * wide);
    double *yabs = (double *)malloc(sizeof(double) * wide);
    double *accL = (double *)malloc(sizeof(double) * L);
    double *DL = (double *)malloc(sizeof(double) * L);
    double *accN = (double *)malloc(sizeof(double) * L);
    double *DN = (double *)malloc(sizeof(double) * L);
    int64_t drops = 0;
    if (!xd || !z || !g || !u || !a || !y || !yabs || !accL || !DL || !accN || !DN) { drops = -1; goto done; }

    for (int64_t t = 0; t < T; t++) {
        double *ot = out + t * H;
        double *dt = denom ? denom + t * H : NULL;
        for (int64_t i = 0; i < H; i++) xd[i] = k3o_bf16(x[t * H + i]);
        k3o_bf16_gemv(z, NULL, xd, lat_down, H, L);
        for (int64_t l = 0; l < L; l++) { accL[l] = 0.0; DL[l] = 0.0; }
        for (int64_t j = 0; j < topk; j++) {
            const int32_t e = idx[t * topk + j];
            if (e < 0 || e >= E) { drops++; continue; }
            const int32_t s = slot_of[e];
            if (s < 0) { drops = -1; goto done; }
            k3o_mxfp4_gemv(g, NULL, z, gate_packed + s * gp, gate_scales + s * gs, L, I);
            k3o_mxfp4_gemv(u, NULL, z, up_packed + s * gp, up_scales + s * gs, L, I);
            for (int64_t n = 0; n < I; n++) a[n] = k3o_act(g[n], u[n], act, b1, b2);
            k3o_mxfp4_gemv(y, yabs, a, down_packed + s * dp, down_scales + s * ds, I, L);
            const double wj = (double)w[t * topk + j];
            for (int64_t l = 0; l < L; l++) {
                accL[l] += wj * y[l];
                DL[l] += fabs(wj) * yabs[l];
            }
        }
        if (norm) {
            double ss = 0.0, cross = 0.0;
            for (int64_t l = 0; l < L; l++) { ss += accL[l] * accL[l]; cross += fabs(accL[l]) * DL[l]; }
            const double inv = k3o_rmsnorm(accN, accL, gamma, L, eps);
            for (int64_t l = 0; l < L; l++) {
                const double gl = gamma ? fabs((double)gamma[l]) : 1.0;
                DN[l] = inv * gl * DL[l] + (ss > 0.0 ? fabs(accN[l]) * cross / ss : 0.0);
            }
        } else {
            for (int64_t l = 0; l < L; l++) { accN[l] = accL[l]; DN[l] = DL[l]; }
        }
        k3o_bf16_gemv(ot, NULL, accN, lat_up, L, H);
        if (dt) {
            for (int64_t o = 0; o < H; o++) {
                double d = 0.0;
                for (int64_t l = 0; l < L; l++) d += fabs(k3o_bf16(lat_up[o * L + l])) * DN[l];
                dt[o] = d;
            }
        }
        if (Is > 0) {
            k3o_bf16_gemv(g, NULL, xd, sh_gate, H, Is);
            k3o_bf16_gemv(u, NULL, xd, sh_up, H, Is);
            for (int64_t n = 0; n < Is; n++) a[n] = k3o_act(g[n], u[n], act, b1, b2);
            k3o_bf16_gemv(y, yabs, a, sh_down, Is, H);
            for (int64_t o = 0; o < H; o++) {
                ot[o] += y[o];
                if (dt) dt[o] += yabs[o];
            }
        }
    }
done:
    free(xd); free(z); free(g); free(u); free(a); free(y); free(yabs);
    free(accL); free(DL); free(accN); free(DN);
    return drops;
}

/* Number of OpenMP threads the oracle's parallel loops use (0 without OpenMP). */
int k3o_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 0;
#endif
}

/* fp32 -> bf16 by its definition: of the two bf16 values around v (the
 * truncation toward zero and the next value away from zero) the nearer one,
 * and on a tie the one whose last bit is 0. Finite v below the bf16 maximum. */
uint16_t k3o_bf16_rne(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    const uint16_t toward = (uint16_t)(u >> 16), away = (uint16_t)(toward + 1);
    const double dt = fabs((double)v - k3o_bf16(toward)), da = fabs(k3o_bf16(away) - (double)v);
    if (dt < da) return toward;
    if (da < dt) return away;
    return (toward & 1) ? away : toward;
}

/* The pre-MoE norm (decoder-layer listing: hin = k3_rmsnorm(h, post_norm);
 * §5 k3_rmsnorm as printed): for each of T rows of n floats,
 *   ss  = sum_i (double)h_i * (double)h_i        (index order, double)
 *   inv = (float)(1 / sqrt(ss / n + eps))         epsilon inside the root
 *   v_i = (h_i * inv) * gamma_i                   two float products
 *   x_i = bf16_RNE(v_i)                           the layer's bf16 token */
void k3o_prenorm_bf16(uint16_t *x, const float *h, const float *gamma, int64_t T, int64_t n, float eps)
{
    for (int64_t t = 0; t < T; t++) {
        const float *ht = h + t * n;
        double ss = 0.0;
        for (int64_t i = 0; i < n; i++) ss += (double)ht[i] * (double)ht[i];
        const float inv = (float)(1.0 / sqrt(ss / (double)n + (double)eps));
        for (int64_t i = 0; i < n; i++) {
            const float p = ht[i] * inv;
            const float v = p * gamma[i];
            x[t * n + i] = k3o_bf16_rne(v);
        }
    }
}
