// gfx950 (MI355X, CDNA4) kernels of the sigmoid-routed MXFP4 expert layer.
//
// What is computed follows the "kimi-k3-in-c" README: §9 "Picking 16 experts
// of 896" (k3_router, k3_moe, k3_situ_glu) and §4 "Reduction one: the experts
// already ship at half a byte" (MXFP4: E2M1 nibbles, one E8M0 scale per 32
// weights, low nibble = even weight, scale byte 255 drops its group).
//
// Design (MI355X-first, not the README's CPU loop):
//  * Expert weights go from HBM straight into the fp4 A operand of the
//    scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4, in the storage layout:
//    lane l of a wave takes 16 bytes = one 32-weight block of row (l % 16),
//    K-block (l / 16), plus that block's E8M0 byte as the lane's A scale.
//    Nothing is dequantised, nothing is repacked, no weight touches LDS.
//  * Activations are the fp8 (e4m3) B operand, as a short expansion
//    x = sum_t 2^(S_t) * q_t with one E8M0 scale per 32-element block per
//    term (4 terms for a bf16 token vector and for an fp32 expert
//    activation). Each term is a separate B column, so one MFMA yields every
//    term's dot product and the terms are added in fp32 afterwards.
//  * The fp8 B operand of this instruction holds, in lane group g = l / 16,
//    K elements [16g, 16g+16) in bytes 0..15 and [64+16g, 64+16g+16) in
//    bytes 16..31; its scale for K-block g comes from lane group g.
//  * Measured on MI355X: the instruction sums each run of 16 consecutive K
//    products to about 14 significant bits below the largest product of the
//    run, then accumulates runs in fp32. Products of fp4 weights with e4m3
//    values spanning at most 7 binades fit that window exactly, so every term
//    keeps only the elements within 6 binades of its block maximum; smaller
//    elements stay in the remainder for the next term. With 4 terms a bf16
//    block is represented exactly and an fp32 block to ~2^-19 of its maximum.
//  * The router sums exact bf16 products in fp64 and takes its decision in
//    fp32, as the README's k3_router does.
//  * The combine sums expert outputs in router order inside one workgroup,
//    with no atomics, so the output is bitwise reproducible.
#include <math.h>

#include "k3moe_internal.h"

namespace k3moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i &a, const v8i &b, v4f c, int sa, int sb)
{
    // A format 4 = fp4 (e2m1), B format 0 = fp8 (e4m3); scale bytes in byte 0.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i a_operand(u4 v) { return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

__device__ __forceinline__ v8i b_operand(u4 lo, u4 hi)
{
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Gated activation (README §9, k3_situ_glu): SiTU-GLU or SwiGLU, fp32.
__device__ __forceinline__ float act_fn(float g, float u, int kind, float b1, float b2)
{
    const float sg = 1.0f / (1.0f + expf(-g));
    if (kind == K3MOE_ACT_SITU) return (b1 * tanhf(g / b1) * sg) * (b2 * tanhf(u / b2));
    return g * sg * u;
}

// Split this lane's value into NT e4m3 terms; the 32 lanes of a half-wave
// form one 32-element block and share one E8M0 scale per term. The scale
// puts the block's largest remainder in [224, 448]; a term takes only the
// elements within 6 binades of that maximum (the rest stay in the remainder)
// and each term's rounding error is carried exactly into the next term.
template <int NT>
__device__ __forceinline__ void split_e4m3_32(float v, int (&code)[NT], int (&sbyte)[NT])
{
    float r = v;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = fabsf(r);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        int S = 0;
        float keep_min = INFINITY;
        if (m > 0.0f) {
            int ex;
            frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
            S = ex - 9;      // m / 2^S in [256, 512)
            if (ldexpf(m, -S) > 448.0f) S += 1;
            if (S < -127) S = -127;
            frexpf(ldexpf(m, -S), &ex);
            keep_min = ldexpf(1.0f, ex - 7);  // 6 binades below the block maximum
        }
        const float q = ldexpf(r, -S);
        int c = 0;
        if (fabsf(q) >= keep_min) {
            c = __builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xff;
            r -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(c, 0), S);
        }
        code[t] = c;
        sbyte[t] = S + 127;
    }
}

// ---------------------------------------------------------------------------
// Router (README §9, k3_router). One wave per (expert, token): 16-byte loads
// of the router row and the token, exact bf16 products summed in fp64, a
// fixed-order butterfly across the wave. Lane 0 then forms the fp32 logit,
// the fp32 score (sigmoid evaluated in fp64, rounded once) and the fp32
// selection score.
__global__ __launch_bounds__(256) void k_router(const uint16_t *__restrict__ x,
                                                const uint16_t *__restrict__ Wr,
                                                const float *__restrict__ bias, int H, int E,
                                                float *__restrict__ sc, float *__restrict__ ch,
                                                float *__restrict__ logits)
{
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = blockIdx.y;
    if (e >= E) return;
    const uint16_t *wr = Wr + (size_t)e * H;
    const uint16_t *xr = x + (size_t)t * H;
    double acc = 0.0;
    for (int i = lane * 8; i < H; i += 512) {
        const u4 wv = *reinterpret_cast<const u4 *>(wr + i);
        const u4 xv = *reinterpret_cast<const u4 *>(xr + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = fma((double)bf16f(wv[q] & 0xffffu), (double)bf16f(xv[q] & 0xffffu), acc);
            acc = fma((double)bf16f(wv[q] >> 16), (double)bf16f(xv[q] >> 16), acc);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) {
        const float l32 = (float)acc;
        const float s = (float)(1.0 / (1.0 + exp(-(double)l32)));
        const size_t o = (size_t)t * E + e;
        sc[o] = s;
        ch[o] = s + (bias ? bias[e] : 0.0f);
        if (logits) logits[o] = l32;
    }
}

// Top-k by repeated maximum (README §9): one wave per token; lane l owns
// experts l, l+64, ...; the order is (ch descending, expert ascending), so a
// tie goes to the lower index. NaN selection scores rank as -inf. Weights
// are the unbiased scores, renormalised in router order, then scaled.
__global__ __launch_bounds__(64) void k_topk(const float *__restrict__ sc,
                                             const float *__restrict__ ch, int E, int K,
                                             int renorm, float rscale, int32_t *__restrict__ idx,
                                             float *__restrict__ w)
{
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    const float *c = ch + (size_t)t * E;
    uint64_t taken = 0;
    int mine = 0;
    for (int j = 0; j < K; ++j) {
        float bv = 0.0f;
        int bi = -1;
        int q = 0;
        for (int e = lane; e < E; e += 64, ++q) {
            if ((taken >> q) & 1ull) continue;
            float v = c[e];
            if (v != v) v = -INFINITY;
            if (bi < 0 || v > bv) {
                bv = v;
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oi = __shfl_xor(bi, o);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
        if (lane == j) mine = bi;
    }
    __shared__ float wj[kMaxTopk];
    __shared__ float ssum;
    if (lane < K) wj[lane] = sc[(size_t)t * E + mine];
    __syncthreads();
    if (lane == 0) {
        float s = 0.0f;
        for (int j = 0; j < K; ++j) s += wj[j];
        ssum = s;
    }
    __syncthreads();
    if (lane < K) {
        float v = wj[lane];
        if (renorm && ssum > 0.0f) v /= ssum;
        v *= rscale;
        idx[(size_t)t * K + lane] = mine;
        w[(size_t)t * K + lane] = v;
    }
}

// ---------------------------------------------------------------------------
// Token activations -> kXTerms e4m3 terms per element, one E8M0 scale per term per
// 32-element block. Thread per element; a half-wave is one block.
__global__ __launch_bounds__(256) void k_xsplit(const uint16_t *__restrict__ x, int64_t n, int H,
                                                uint8_t *__restrict__ xq, uint8_t *__restrict__ xs)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;  // n is a multiple of 32: whole half-waves leave together
    const int64_t t = i / H;
    const int col = (int)(i - t * H);
    int code[kXTerms], sb[kXTerms];
    split_e4m3_32<kXTerms>(bf16f(x[i]), code, sb);
#pragma unroll
    for (int term = 0; term < kXTerms; ++term) {
        xq[(t * kXTerms + term) * H + col] = (uint8_t)code[term];
        if ((threadIdx.x & 31) == 0) xs[(t * kXTerms + term) * (H >> 5) + (col >> 5)] = (uint8_t)sb[term];
    }
}

// ---------------------------------------------------------------------------
// Token -> expert permutation: a stable counting sort of the T*k assignments
// a = t*k + j by expert, in (t, j) order. Outputs the active experts in
// ascending id, their start offsets, and the sorted assignment list.
// Out-of-range ids are left out (the combine counts them).

// Exclusive scan, in place, of v[0..n) (n <= 4096) by a 1024-thread block;
// returns the total.
__device__ int block_exclusive_scan(int *v, int n)
{
    __shared__ int wsum[16];
    __shared__ int total_sh;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (n + 1023) >> 10;
    int loc[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * per + q;
        loc[q] = (q < per && i < n) ? v[i] : 0;
        s += loc[q];
    }
    int inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int k = 0; k < 16; ++k) {
            const int c = wsum[k];
            wsum[k] = run;
            run += c;
        }
        total_sh = run;
    }
    __syncthreads();
    int base = wsum[wv] + inc - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * per + q;
        if (q < per && i < n) {
            v[i] = base;
            base += loc[q];
        }
    }
    __syncthreads();
    const int total = total_sh;
    __syncthreads();
    return total;
}

// From per-expert counts cnt[e] (LDS): offsets (into off[]), the active list.
__device__ void build_active(const int *cnt, int *off, int *flag, int E, int32_t *active_n,
                             int32_t *active_e, int32_t *active_off)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) {
        off[e] = cnt[e];
        flag[e] = cnt[e] > 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(off, E);
    const int nact = block_exclusive_scan(flag, E);
    for (int e = tid; e < E; e += 1024) {
        if (cnt[e] > 0) {
            active_e[flag[e]] = e;
            active_off[flag[e]] = off[e];
        }
    }
    if (tid == 0) {
        *active_n = nact;
        active_off[nact] = total;
    }
    __syncthreads();
}

// Whole permutation in one block, for T <= kPermChunk.
__global__ __launch_bounds__(1024) void k_perm_single(const int32_t *__restrict__ idx, int T, int K,
                                                      int E, int32_t *active_n, int32_t *active_e,
                                                      int32_t *active_off, int32_t *sorted)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int off[kMaxExperts];
    __shared__ int flag[kMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < T * K; a += 1024) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    build_active(cnt, off, flag, E, active_n, active_e, active_off);
    if (tid < 64) {  // one wave, tokens in order: stable
        for (int t = 0; t < T; ++t)
            for (int j = tid; j < K; j += 64) {
                const int e = idx[t * K + j];
                if (e >= 0 && e < E) sorted[atomicAdd(&off[e], 1)] = t * K + j;
            }
    }
}

// Multi-chunk permutation, phase 1: per-chunk expert counts.
__global__ __launch_bounds__(256) void k_perm_hist(const int32_t *__restrict__ idx, int T, int K,
                                                   int E, int32_t *__restrict__ chunk_cnt)
{
    __shared__ int h[kMaxExperts];
    const int c = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int t0 = c * kPermChunk, t1 = min(T, t0 + kPermChunk);
    for (int a = t0 * K + tid; a < t1 * K; a += 256) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) chunk_cnt[(size_t)c * E + e] = h[e];
}

// Phase 2: totals, offsets, active list; chunk counts become chunk bases.
__global__ __launch_bounds__(1024) void k_perm_scan(int nchunks, int E, int32_t *__restrict__ chunk_cnt,
                                                    int32_t *active_n, int32_t *active_e,
                                                    int32_t *active_off)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int off[kMaxExperts];
    __shared__ int flag[kMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) {
        int s = 0;
        for (int c = 0; c < nchunks; ++c) s += chunk_cnt[(size_t)c * E + e];
        cnt[e] = s;
    }
    __syncthreads();
    build_active(cnt, off, flag, E, active_n, active_e, active_off);
    for (int e = tid; e < E; e += 1024) {
        int run = off[e];
        for (int c = 0; c < nchunks; ++c) {
            const int v = chunk_cnt[(size_t)c * E + e];
            chunk_cnt[(size_t)c * E + e] = run;
            run += v;
        }
    }
}

// Phase 3: stable scatter, one wave per chunk, tokens in order.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t *__restrict__ idx, int T, int K,
                                                     int E, const int32_t *__restrict__ chunk_base,
                                                     int32_t *__restrict__ sorted)
{
    __shared__ int cur[kMaxExperts];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) cur[e] = chunk_base[(size_t)c * E + e];
    __syncthreads();
    const int t0 = c * kPermChunk, t1 = min(T, t0 + kPermChunk);
    for (int t = t0; t < t1; ++t)
        for (int j = lane; j < K; j += 64) {
            const int e = idx[t * K + j];
            if (e >= 0 && e < E) sorted[atomicAdd(&cur[e], 1)] = t * K + j;
        }
}

// ---------------------------------------------------------------------------
// Gate/up projections + activation for the routed experts (README §9, k3_moe
// step 3, first half). One workgroup per (active expert, 32-row tile of I);
// its 4 waves split the K steps (128 elements each) round-robin and meet in
// LDS. Per K step a wave loads 4 A fragments (gate/up x two 16-row halves)
// and one B fragment carrying up to 4 tokens x 4 terms, and issues 4 MFMAs.
// The epilogue adds the term columns, applies the activation, and writes
// the activation as 4 e4m3 terms (with E8M0 scales) for the down projection.
struct GateUpParams {
    const uint8_t *gp, *gs, *up, *us;
    int64_t g_sp, g_ss, u_sp, u_ss;
    int H, I, K, act;
    float b1, b2;
    const uint8_t *xq, *xs;
    const int32_t *active_n, *active_e, *active_off, *sorted;
    uint8_t *aq, *as;
};

__global__ __launch_bounds__(256) void k_gateup(GateUpParams p)
{
    const int RT = p.I >> 5;
    const int slot = blockIdx.x / RT;
    const int rt = blockIdx.x - slot * RT;
    if (slot >= *p.active_n) return;
    const int e = p.active_e[slot];
    const int a0 = p.active_off[slot], a1 = p.active_off[slot + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int H = p.H, KS = H >> 7;
    const int64_t rowb = H >> 1, rows = H >> 5;

    const uint8_t *ap[4];
    const uint8_t *asp[4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t row = (int64_t)rt * 32 + h * 16 + rl;
            ap[m * 2 + h] = (m ? p.up + e * p.u_sp : p.gp + e * p.g_sp) + row * rowb + grp * 16;
            asp[m * 2 + h] = (m ? p.us + e * p.u_ss : p.gs + e * p.g_ss) + row * rows + grp;
        }

    __shared__ float red[4][4][4][64];  // [wave][tile][reg][lane]

    constexpr int kTok = 16 / kXTerms;  // tokens per B fragment
    for (int g0 = a0; g0 < a1; g0 += kTok) {
        const int ntok = min(kTok, a1 - g0);
        const int col = lane & 15, s = col / kXTerms, term = col - kXTerms * s;
        const bool bvalid = (s < kTok) && (s < ntok);
        const uint8_t *xb = p.xq;
        const uint8_t *xsb = p.xs;
        if (bvalid) {
            const int64_t tok = p.sorted[g0 + s] / p.K;
            xb += (tok * kXTerms + term) * H + grp * 16;
            xsb += (tok * kXTerms + term) * (H >> 5) + grp;
        }
        v4f acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

        for (int st = wave; st < KS; st += 4) {
            u4 av[4];
            int sa[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                av[q] = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(ap[q] + st * 64));
                sa[q] = asp[q][st * 4];
            }
            u4 lo = u4{0u, 0u, 0u, 0u}, hi = u4{0u, 0u, 0u, 0u};
            int sb = 127;
            if (bvalid) {
                lo = *reinterpret_cast<const u4 *>(xb + st * 128);
                hi = *reinterpret_cast<const u4 *>(xb + st * 128 + 64);
                sb = xsb[st * 4];
            }
            const v8i B = b_operand(lo, hi);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (sa[q] == 255) {  // scale byte 255: the 32-group drops out
                    av[q] = u4{0u, 0u, 0u, 0u};
                    sa[q] = 127;
                }
                acc[q] = mfma_fp4_fp8(a_operand(av[q]), B, acc[q], sa[q], sb);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][q][r][lane] = acc[q][r];
        __syncthreads();
        {
            const int q = threadIdx.x >> 6;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[0][q][r][lane] = ((red[0][q][r][lane] + red[1][q][r][lane]) + red[2][q][r][lane]) +
                                     red[3][q][r][lane];
        }
        __syncthreads();
        if (threadIdx.x < 32 * kTok) {
            const int ts = threadIdx.x >> 5, r = threadIdx.x & 31;
            if (ts < ntok) {  // uniform over each half-wave
                const int h = r >> 4, rho = r & 15;
                const int ln = 16 * (rho >> 2) + kXTerms * ts, rg = rho & 3;
                float g = 0.0f, u = 0.0f;
#pragma unroll
                for (int k = 0; k < kXTerms; ++k) {
                    g += red[0][h][rg][ln + k];
                    u += red[0][2 + h][rg][ln + k];
                }
                const float a = act_fn(g, u, p.act, p.b1, p.b2);
                int code[kATerms], sbt[kATerms];
                split_e4m3_32<kATerms>(a, code, sbt);
                const int64_t asg = p.sorted[g0 + ts];
#pragma unroll
                for (int k = 0; k < kATerms; ++k) {
                    p.aq[(asg * kATerms + k) * p.I + rt * 32 + r] = (uint8_t)code[k];
                    if (r == 0) p.as[(asg * kATerms + k) * (p.I >> 5) + rt] = (uint8_t)sbt[k];
                }
            }
        }
        __syncthreads();
    }
}

// Shared expert gate/up + activation (README §9, k3_moe step 6, first half),
// bf16 weights, fp32 accumulation. One wave per shared row, tokens in turn.
__global__ __launch_bounds__(256) void k_shared_gateup(const uint16_t *__restrict__ x, int T, int H,
                                                       int Is, const uint16_t *__restrict__ S1,
                                                       const uint16_t *__restrict__ S3, int act,
                                                       float b1, float b2, float *__restrict__ ash)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= Is) return;
    const uint16_t *g = S1 + (size_t)r * H;
    const uint16_t *u = S3 + (size_t)r * H;
    for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (size_t)t * H;
        float ga = 0.0f, ua = 0.0f;
        for (int i = lane * 8; i < H; i += 512) {
            const u4 gv = *reinterpret_cast<const u4 *>(g + i);
            const u4 uv = *reinterpret_cast<const u4 *>(u + i);
            const u4 xv = *reinterpret_cast<const u4 *>(xr + i);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = bf16f(xv[q] & 0xffffu), x1 = bf16f(xv[q] >> 16);
                ga = fmaf(bf16f(gv[q] & 0xffffu), x0, ga);
                ga = fmaf(bf16f(gv[q] >> 16), x1, ga);
                ua = fmaf(bf16f(uv[q] & 0xffffu), x0, ua);
                ua = fmaf(bf16f(uv[q] >> 16), x1, ua);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            ga += __shfl_xor(ga, o);
            ua += __shfl_xor(ua, o);
        }
        if (lane == 0) ash[(size_t)t * Is + r] = act_fn(ga, ua, act, b1, b2);
    }
}

// Down projection + router-order combine + shared expert (README §9, k3_moe
// step 3 second half and step 6). One workgroup per (16-row tile of H,
// token); wave w runs the experts j = w, w+4, ...; each expert's 16 outputs
// land in LDS, then 16 threads sum w_j * y_j in j order and add the shared
// expert's rows. An expert id outside [0, E) contributes zero and is counted.
struct DownParams {
    const uint8_t *dp, *ds;
    int64_t d_sp, d_ss;
    int H, I, E, K, Is;
    const int32_t *idx;
    const float *w;
    const uint8_t *aq, *as;
    const uint16_t *sh_down;
    const float *ash;
    float *out;
    unsigned long long *errors;
};

__global__ __launch_bounds__(256) void k_down(DownParams p)
{
    const int rt = blockIdx.x, t = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int KS = p.I >> 7;
    const int64_t rowb = p.I >> 1, rows = p.I >> 5;
    const int64_t row = (int64_t)rt * 16 + rl;
    __shared__ float ys[kMaxTopk][16];
    __shared__ float sh[16];

    for (int j = wave; j < p.K; j += 4) {
        const int e = p.idx[(size_t)t * p.K + j];
        const bool ok = (e >= 0) && (e < p.E);
        v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        if (ok) {
            const uint8_t *ap = p.dp + (int64_t)e * p.d_sp + row * rowb + grp * 16;
            const uint8_t *asp = p.ds + (int64_t)e * p.d_ss + row * rows + grp;
            const int col = lane & 15;
            const bool bvalid = col < kATerms;
            const int64_t asg = (int64_t)t * p.K + j;
            const uint8_t *bp = p.aq + (asg * kATerms + (bvalid ? col : 0)) * p.I + grp * 16;
            const uint8_t *bsp = p.as + (asg * kATerms + (bvalid ? col : 0)) * (p.I >> 5) + grp;
            for (int st = 0; st < KS; ++st) {
                u4 av = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(ap + st * 64));
                int sa = asp[st * 4];
                if (sa == 255) {
                    av = u4{0u, 0u, 0u, 0u};
                    sa = 127;
                }
                u4 lo = u4{0u, 0u, 0u, 0u}, hi = u4{0u, 0u, 0u, 0u};
                int sb = 127;
                if (bvalid) {
                    lo = *reinterpret_cast<const u4 *>(bp + st * 128);
                    hi = *reinterpret_cast<const u4 *>(bp + st * 128 + 64);
                    sb = bsp[st * 4];
                }
                acc = mfma_fp4_fp8(a_operand(av), b_operand(lo, hi), acc, sa, sb);
            }
        } else if (rt == 0 && lane == 0) {
            atomicAdd(p.errors, 1ull);
        }
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = acc[r] + __shfl_xor(acc[r], 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = y[r] + __shfl_xor(y[r], 2);
        if ((lane & 15) == 0) {
            const int q = lane >> 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) ys[j][4 * q + r] = y[r];
        }
    }
    if (p.Is > 0) {
        const float *a = p.ash + (size_t)t * p.Is;
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t orow = (int64_t)rt * 16 + wave * 4 + rr;
            const uint16_t *srow = p.sh_down + orow * p.Is;
            float acc = 0.0f;
            for (int i = lane * 8; i < p.Is; i += 512) {
                const u4 wv = *reinterpret_cast<const u4 *>(srow + i);
                const float4 a0 = *reinterpret_cast<const float4 *>(a + i);
                const float4 a1 = *reinterpret_cast<const float4 *>(a + i + 4);
                acc = fmaf(bf16f(wv[0] & 0xffffu), a0.x, acc);
                acc = fmaf(bf16f(wv[0] >> 16), a0.y, acc);
                acc = fmaf(bf16f(wv[1] & 0xffffu), a0.z, acc);
                acc = fmaf(bf16f(wv[1] >> 16), a0.w, acc);
                acc = fmaf(bf16f(wv[2] & 0xffffu), a1.x, acc);
                acc = fmaf(bf16f(wv[2] >> 16), a1.y, acc);
                acc = fmaf(bf16f(wv[3] & 0xffffu), a1.z, acc);
                acc = fmaf(bf16f(wv[3] >> 16), a1.w, acc);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
            if (lane == 0) sh[wave * 4 + rr] = acc;
        }
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        float o = 0.0f;
        for (int j = 0; j < p.K; ++j) o = fmaf(p.w[(size_t)t * p.K + j], ys[j][threadIdx.x], o);
        if (p.Is > 0) o += sh[threadIdx.x];
        p.out[(size_t)t * p.H + rt * 16 + threadIdx.x] = o;
    }
}

}  // namespace

hipError_t launch_route(const LayerView &L, const uint16_t *x, int T, int32_t *idx, float *w,
                        float *logits, char *ws, const WsLayout &lay, hipStream_t s, Profiler *prof)
{
    float *sc = reinterpret_cast<float *>(ws + lay.sc);
    float *ch = reinterpret_cast<float *>(ws + lay.ch);
    {
        StageMark m(prof, K3MOE_STAGE_ROUTER, s);
        k_router<<<dim3((L.E + 3) / 4, T), 256, 0, s>>>(x, L.router_w, L.router_bias, L.H, L.E, sc,
                                                        ch, logits);
    }
    {
        StageMark m(prof, K3MOE_STAGE_TOPK, s);
        k_topk<<<T, 64, 0, s>>>(sc, ch, L.E, L.K, L.renorm, L.routed_scale, idx, w);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const LayerView &L, const uint16_t *x, int T, const int32_t *idx,
                          const float *w, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                          Profiler *prof)
{
    uint8_t *xq = reinterpret_cast<uint8_t *>(ws + lay.xq);
    uint8_t *xs = reinterpret_cast<uint8_t *>(ws + lay.xs);
    int32_t *chunk_cnt = reinterpret_cast<int32_t *>(ws + lay.chunk_cnt);
    int32_t *active_n = reinterpret_cast<int32_t *>(ws + lay.active_n);
    int32_t *active_e = reinterpret_cast<int32_t *>(ws + lay.active_e);
    int32_t *active_off = reinterpret_cast<int32_t *>(ws + lay.active_off);
    int32_t *sorted = reinterpret_cast<int32_t *>(ws + lay.sorted);
    uint8_t *aq = reinterpret_cast<uint8_t *>(ws + lay.aq);
    uint8_t *as = reinterpret_cast<uint8_t *>(ws + lay.as);
    float *ash = reinterpret_cast<float *>(ws + lay.ash);

    const int64_t n = (int64_t)T * L.H;
    {
        StageMark m(prof, K3MOE_STAGE_XSPLIT, s);
        k_xsplit<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, n, L.H, xq, xs);
    }

    const int nchunks = (T + kPermChunk - 1) / kPermChunk;
    StageMark *pm = new StageMark(prof, K3MOE_STAGE_PERM, s);
    if (nchunks == 1) {
        k_perm_single<<<1, 1024, 0, s>>>(idx, T, L.K, L.E, active_n, active_e, active_off, sorted);
    } else {
        k_perm_hist<<<nchunks, 256, 0, s>>>(idx, T, L.K, L.E, chunk_cnt);
        k_perm_scan<<<1, 1024, 0, s>>>(nchunks, L.E, chunk_cnt, active_n, active_e, active_off);
        k_perm_scatter<<<nchunks, 64, 0, s>>>(idx, T, L.K, L.E, chunk_cnt, sorted);
    }
    delete pm;

    GateUpParams gp;
    gp.gp = L.gp;
    gp.gs = L.gs;
    gp.up = L.up;
    gp.us = L.us;
    gp.g_sp = L.g_sp;
    gp.g_ss = L.g_ss;
    gp.u_sp = L.u_sp;
    gp.u_ss = L.u_ss;
    gp.H = L.H;
    gp.I = L.I;
    gp.K = L.K;
    gp.act = L.act;
    gp.b1 = L.b1;
    gp.b2 = L.b2;
    gp.xq = xq;
    gp.xs = xs;
    gp.active_n = active_n;
    gp.active_e = active_e;
    gp.active_off = active_off;
    gp.sorted = sorted;
    gp.aq = aq;
    gp.as = as;
    const int64_t max_active = std::min<int64_t>(L.E, (int64_t)T * L.K);
    {
        StageMark m(prof, K3MOE_STAGE_GATEUP, s);
        k_gateup<<<(unsigned)(max_active * (L.I / 32)), 256, 0, s>>>(gp);
    }
    if (L.Is > 0) {
        StageMark m(prof, K3MOE_STAGE_SHARED_GATEUP, s);
        k_shared_gateup<<<(L.Is + 3) / 4, 256, 0, s>>>(x, T, L.H, L.Is, L.sh_gate, L.sh_up, L.act,
                                                        L.b1, L.b2, ash);
    }

    DownParams dp;
    dp.dp = L.dp;
    dp.ds = L.ds;
    dp.d_sp = L.d_sp;
    dp.d_ss = L.d_ss;
    dp.H = L.H;
    dp.I = L.I;
    dp.E = L.E;
    dp.K = L.K;
    dp.Is = L.Is;
    dp.idx = idx;
    dp.w = w;
    dp.aq = aq;
    dp.as = as;
    dp.sh_down = L.sh_down;
    dp.ash = ash;
    dp.out = out;
    dp.errors = L.errors;
    {
        StageMark m(prof, K3MOE_STAGE_DOWN, s);
        k_down<<<dim3(L.H / 16, T), 256, 0, s>>>(dp);
    }
    return hipGetLastError();
}

}  // namespace k3moe
