// gfx950 (MI355X, CDNA4) kernels of the sigmoid-routed MXFP4 expert layer.
//
// What is computed follows the "kimi-k3-in-c" README: §9 "Picking 16 experts
// of 896" (k3_router, k3_moe, k3_situ_glu) and §4 "Reduction one: the experts
// already ship at half a byte" (MXFP4: E2M1 nibbles, one E8M0 scale per 32
// weights, low nibble = even weight, scale byte 255 drops its group).
//
// Design (MI355X-first, not the README's CPU loop):
//  * Single-token gate/up (k_gateup_dec): weights go from HBM straight into
//    registers, lane l of a wave taking 16 bytes = one 32-weight block of
//    row (l % 16), K-block (l / 16); they are expanded to bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp4 applies the E8M0 scale exactly) and
//    multiplied on v_mfma_f32_16x16x32_bf16 with the bf16 token (one or two
//    planes) staged in LDS: every product exact, fp32 accumulation.
//  * Single-token down (k_down_dec): the weight bytes are the fp4 A operand
//    of the scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 as loaded, the
//    E8M0 byte the lane's A scale; nothing is dequantised or repacked and no
//    weight touches LDS. The fp32 activation is the fp8 (e4m3) B operand as
//    a short expansion a = sum_t 2^(S_t) * q_t with one E8M0 scale per
//    32-element block per term (kATerms = 4 terms). Each term is a separate
//    B column, so one MFMA yields every term's dot product and the terms are
//    added in fp32 afterwards.
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

#include <type_traits>

#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

// Router (README §9, k3_router). One wave per (expert, token): 16-byte loads
// of the router row and the token, exact bf16 products summed in fp64, a
// fixed-order butterfly across the wave. Lane 0 then forms the fp32 logit,
// the fp32 score (sigmoid evaluated in fp64, rounded once) and the fp32
// selection score. NT: one token, so each router row is read once (a
// streaming load); with more tokens the rows are read once per token.
template <bool NT>
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
    constexpr int CH = 14;  // 512-element slices whose loads are issued together
    for (int i0 = lane * 8; i0 < H; i0 += 512 * CH) {
        u4 wv[CH], xv[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = i0 + 512 * c;
            if constexpr (NT)
                wv[c] = i < H ? ld16_stream(wr + i) : u4{0u, 0u, 0u, 0u};
            else
                wv[c] = i < H ? *reinterpret_cast<const u4 *>(wr + i) : u4{0u, 0u, 0u, 0u};
            xv[c] = i < H ? *reinterpret_cast<const u4 *>(xr + i) : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fma((double)bf16f(wv[c][q] & 0xffffu), (double)bf16f(xv[c][q] & 0xffffu), acc);
                acc = fma((double)bf16f(wv[c][q] >> 16), (double)bf16f(xv[c][q] >> 16), acc);
            }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) router_finish(acc, t, e, E, bias, sc, ch, logits);
}

// Batched router: logits = Wr X^T. Each 32-element chunk of the hidden
// dimension is one v_mfma_f32_16x16x32_bf16 per 16 x 16 tile, started from
// zero: its 32 bf16 products are exact in fp32 and the instruction sums them
// in fp32; the chunk sums are then added in fp64, in chunk order. The logit
// is therefore the fp64 sum of fp32 sums of 32 exact products each, not of
// the products themselves: on N(0,1) tokens and N(0, 1/H) router rows at
// H = 7168 it stays within about 2^-22 of the exact sum, far inside the
// selection-score margin the routes are compared with.
// A block takes 128 experts x 32 WT tokens over one slice of the hidden
// dimension (the grid's z), 64 elements per stage: the stage's rows (experts
// first, then tokens) go through double-buffered LDS, eight threads per
// row's 128 bytes, so every row is read from the caches once per block.
// Wave (we, wt) computes experts 32 we .. 32 we + 31 of tokens 32 wt ..
// 32 wt + 31 (2 x 2 MFMA tiles); lane group g reads elements 8g .. 8g + 7 of
// a chunk, the MFMA operand layout. One slice: finished in place; several:
// fp64 partial sums [slice][T][E], added in slice order by k_router_reduce.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int kRtE = 128;              // experts per block
constexpr int kRtK = 64;               // hidden elements per stage
constexpr int kRtRow = 2 * kRtK + 16;  // LDS bytes per staged row (16 of padding)
constexpr int kRtDepth = 3;            // stages whose loads are in flight

template <int WT>
__host__ __device__ constexpr int rt_lds_bytes()
{
    return 2 * (kRtE + 32 * WT) * kRtRow;
}

template <int WT>
__global__ __launch_bounds__(256 * WT) void k_router_mm(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ Wr, int T, int H, int E,
                                                        int kspan, double *__restrict__ part,
                                                        const float *__restrict__ bias, float *__restrict__ sc,
                                                        float *__restrict__ ch, float *__restrict__ logits)
{
    extern __shared__ __align__(16) uint8_t rt_l[];
    constexpr int TT = 32 * WT, NROW = kRtE + TT, NT = 256 * WT;
    constexpr int NU = NROW * (kRtK / 8);  // 16-byte pieces per stage
    static_assert(NU % NT == 0, "whole pieces per thread");
    constexpr int NQ = NU / NT;
    constexpr int BUF = NROW * kRtRow;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int we = wave & 3, wt = wave >> 2, g = lane >> 4, l16 = lane & 15;
    const int eb = blockIdx.x * kRtE, tb = blockIdx.y * TT;
    const int k0 = blockIdx.z * kspan, nst = (min(H, k0 + kspan) - k0) / kRtK;

    // piece v = tid + NT q: staged row v / 8 (rows past E or T repeat the
    // last one; their results are never stored), 16-byte segment v % 8
    const uint16_t *src[NQ];
    uint32_t dst[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int v = tid + NT * q, row = v >> 3, seg = v & 7;
        src[q] = row < kRtE ? Wr + (size_t)min(eb + row, E - 1) * H + k0 + 8 * seg
                            : x + (size_t)min(tb + row - kRtE, T - 1) * H + k0 + 8 * seg;
        dst[q] = (uint32_t)(row * kRtRow + 16 * seg);
    }
    // three stages in flight: register sets st[0..2] rotate (named, so the
    // compiler's wait counts follow the rotation); loads past the last stage
    // repeat it (never computed)
    u4 st[kRtDepth][NQ];
    auto gload = [&](int s, u4 (&r)[NQ]) {
        const int sc = min(s, nst - 1);
#pragma unroll
        for (int q = 0; q < NQ; ++q) r[q] = *reinterpret_cast<const u4 *>(src[q] + kRtK * sc);
    };
    auto lstore = [&](int buf, const u4 (&r)[NQ]) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) *reinterpret_cast<u4 *>(rt_l + buf * BUF + dst[q]) = r[q];
    };
    v4d acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
    auto compute = [&](int buf) {
        const uint8_t *Ab = rt_l + buf * BUF + (32 * we + l16) * kRtRow;
        const uint8_t *Bb = rt_l + buf * BUF + (kRtE + 32 * wt + l16) * kRtRow;
#pragma unroll
        for (int c = 0; c < kRtK / 32; ++c) {
            const int kb = 64 * c + 16 * g;  // bytes: elements 32 c + 8 g .. + 7
            bf8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = as_bf8(*reinterpret_cast<const u4 *>(Ab + 16 * i * kRtRow + kb));
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = as_bf8(*reinterpret_cast<const u4 *>(Bb + 16 * j * kRtRow + kb));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const v4f cs = mfma_bf16(a[i], b[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += (double)cs[r];
                }
        }
    };
#pragma unroll
    for (int d = 0; d < kRtDepth; ++d) gload(d, st[d]);
    lstore(0, st[0]);
    __syncthreads();
    // stage i: st[i % 3] (already in LDS buffer i % 2) takes stage i + 3;
    // st[(i + 1) % 3] goes to the other buffer
    for (int s = 0; s < nst; s += kRtDepth) {
#pragma unroll
        for (int u = 0; u < kRtDepth; ++u) {
            if (s + u < nst) {  // uniform
                gload(s + u + kRtDepth, st[u]);
                compute((s + u) & 1);
                lstore((s + u + 1) & 1, st[(u + 1) % kRtDepth]);
                __syncthreads();
            }
        }
    }
    // tile (i, j): lane l holds rows 4 (l / 16) + r of column l % 16 in result
    // register r, i.e. expert 32 we + 16 i + 4 g + r of token 32 wt + 16 j + l16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = tb + 32 * wt + 16 * j + l16;
            if (t >= T) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = eb + 32 * we + 16 * i + 4 * g + r;
                if (e >= E) continue;
                if (part)
                    part[((size_t)blockIdx.z * T + t) * E + e] = acc[i][j][r];
                else
                    router_finish(acc[i][j][r], t, e, E, bias, sc, ch, logits);
            }
        }
}

// Slice partial sums -> logits, in slice order (eight slices' loads in flight
// at a time).
__global__ __launch_bounds__(256) void k_router_reduce(const double *__restrict__ part, int S, int T, int E,
                                                       const float *__restrict__ bias, float *__restrict__ sc,
                                                       float *__restrict__ ch, float *__restrict__ logits)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x, n = (int64_t)T * E;
    if (i >= n) return;
    double acc = part[i];
    for (int s0 = 1; s0 < S; s0 += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s0 + u < S ? part[(size_t)(s0 + u) * n + i] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) acc += v[u];
    }
    const int t = (int)(i / E);
    router_finish(acc, t, (int)(i - (int64_t)t * E), E, bias, sc, ch, logits);
}

// Top-k (README §9): one wave per token (topk_wave).
template <int NQ, bool V4>
__global__ __launch_bounds__(64) void k_topk(const float *__restrict__ sc, const float *__restrict__ ch,
                                             int E, int K, int renorm, float rscale,
                                             int32_t *__restrict__ idx, float *__restrict__ w)
{
    __shared__ TopkLds lds;
    const int t = blockIdx.x, lane = threadIdx.x;
    int pick;
    float wt;
    topk_wave<NQ, V4>(sc + (size_t)t * E, ch + (size_t)t * E, E, K, renorm, rscale, lds, &pick, &wt);
    if (lane < K) {
        w[(size_t)t * K + lane] = wt;
        idx[(size_t)t * K + lane] = pick;
    }
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Token -> expert permutation: a stable counting sort of the T*k assignments
// a = t*k + j by expert, in (t, j) order. Outputs the active experts in
// ascending id, their start offsets, and the sorted assignment list.
// Out-of-range ids are left out (the combine counts them).

// Exclusive scan, in place, of v[0..n) (LDS) by the whole block (blockDim a
// multiple of 64, at most 1024); returns the total.
__device__ int block_exclusive_scan(int *v, int n)
{
    __shared__ int wsum[16];
    __shared__ int total_sh;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    int s = 0;
    for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) s += v[i];
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
        for (int k = 0; k < nt / 64; ++k) {
            const int c = wsum[k];
            wsum[k] = run;
            run += c;
        }
        total_sh = run;
    }
    __syncthreads();
    int base = wsum[wv] + inc - s;
    for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) {
            const int c = v[i];
            v[i] = base;
            base += c;
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
    for (int e = tid; e < E; e += blockDim.x) {
        off[e] = cnt[e];
        flag[e] = cnt[e] > 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(off, E);
    const int nact = block_exclusive_scan(flag, E);
    for (int e = tid; e < E; e += blockDim.x) {
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
__device__ void perm_single(const int32_t *__restrict__ idx, int T, int K, int E, int32_t *active_n,
                            int32_t *active_e, int32_t *active_off, int32_t *sorted)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int off[kMaxExperts];
    __shared__ int flag[kMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < T * K; a += blockDim.x) {
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

// Small batches (T <= kPermChunk): the whole permutation in one block.
__global__ __launch_bounds__(256) void k_perm_small(const int32_t *__restrict__ idx, int T, int K, int E,
                                                    int32_t *active_n, int32_t *active_e,
                                                    int32_t *active_off, int32_t *sorted)
{
    perm_single(idx, T, K, E, active_n, active_e, active_off, sorted);
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
    // a thread per expert walks the chunks in batches of 16 loads in flight
    constexpr int B = 16;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) {
        int s = 0, c = 0;
        for (; c + B <= nchunks; c += B) {
            int v[B];
#pragma unroll
            for (int q = 0; q < B; ++q) v[q] = chunk_cnt[(size_t)(c + q) * E + e];
#pragma unroll
            for (int q = 0; q < B; ++q) s += v[q];
        }
        for (; c < nchunks; ++c) s += chunk_cnt[(size_t)c * E + e];
        cnt[e] = s;
    }
    __syncthreads();
    build_active(cnt, off, flag, E, active_n, active_e, active_off);
    for (int e = tid; e < E; e += 1024) {
        int run = off[e], c = 0;
        for (; c + B <= nchunks; c += B) {
            int v[B];
#pragma unroll
            for (int q = 0; q < B; ++q) v[q] = chunk_cnt[(size_t)(c + q) * E + e];
#pragma unroll
            for (int q = 0; q < B; ++q) {
                chunk_cnt[(size_t)(c + q) * E + e] = run;
                run += v[q];
            }
        }
        for (; c < nchunks; ++c) {
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
// Parameters of the single-token gate/up kernel (below).
struct GateUpParams {
    const uint8_t *gp, *gs, *up, *us;
    int64_t g_sp, g_ss, u_sp, u_ss;
    int H, I, K, E, act, Is;
    float b1, b2;
    const uint16_t *x;      // the token, bf16 [H] (the shared expert's input)
    const uint16_t *xr;     // the routed experts' input, bf16 [Kr] (x for a flat layer; hi of z)
    const uint16_t *xr_lo;  // its lo plane (latent z) or null
    int Kr;                 // routed input width (H, or the latent)
    const int32_t *idx;
    float *act_f;  // fp32 activations [k][I]
    const uint16_t *sh_gate, *sh_up;
    float *ash;
};

// ---------------------------------------------------------------------------
// Single-token path (T = 1). The k assignments are the router slots j
// themselves (slot j takes expert idx[j]), so no permutation is built.

// ---------------------------------------------------------------------------
// Single-token kernels. On MI355X a CU streams weights at ~23-26 GB/s with
// the MFMA operand access pattern, so these grids give every CU the same
// number of bytes: the kernel time is the most loaded CU's time.

// Gate/up, T = 1. Routed work comes in units of (slot, 16-row tile of I),
// gate and up, over the whole K range: 2 weight fragments per K step straight
// from HBM into the MFMA A operand. A block of 4 waves runs 3 units (waves
// 0..2) and a slice of the shared expert's rows (wave 3); with two blocks per
// CU every CU moves the same bytes. The bf16 token planes and the units'
// E8M0 rows are staged in LDS once per block; K is walked in chunks of 4
// steps, double-buffered in registers. The activation is written in fp32
// (act_f[slot][I]); the down kernel expands it into e4m3 terms.
constexpr int kGuDecWaves = 4;                 // waves per block
constexpr int kGuDecMaxUnits = 3;              // routed units per block (waves 0..UNITS-1), at most
constexpr int kGuUnitRows = 16;                // rows per routed unit
constexpr int kGuShMaxRows = 4;                // shared rows per pass of wave 3
constexpr int kXqPad = 64;                     // LDS term-row padding (banks)
constexpr int kScPad = 16;                     // LDS scale-row padding (banks)
constexpr int kGuStgQ = 8;                     // token staging copies per thread (16 B of bf16)
constexpr int kGuStgS = 6;                     // scale-row staging copies per thread

// the routed input (np planes of Kr bf16) and the units' scale rows
__host__ __device__ constexpr int gu_dec_lds_bytes(int Kr, int np)
{
    return 2 * Kr * np + kGuDecMaxUnits * 2 * kGuUnitRows * (Kr / 32 + kScPad);
}

// Wave 3 of a gate/up block: shared rows [r0, r1) of gate and up (bf16,
// fp32 FMA), activation to ash. 512-element slices, 8 elements per lane,
// double-buffered; unconditional clamped loads (a lane past the row end
// multiplies 0).
__device__ void shared_gateup_rows(const GateUpParams &p, int r0, int r1)
{
    const int lane = threadIdx.x & 63;
    const int H = p.H;
    const int NS = (H + 511) >> 9;
    struct Slice {
        u4 w[2 * kGuShMaxRows];  // gate rows, up rows
        u4 x;
    };
    for (int ra = r0; ra < r1; ra += kGuShMaxRows) {
        const int nr = min(kGuShMaxRows, r1 - ra);
        float acc[2 * kGuShMaxRows];
#pragma unroll
        for (int q = 0; q < 2 * kGuShMaxRows; ++q) acc[q] = 0.0f;
        auto load = [&](int sl, Slice &b) {
            const int i = sl * 512 + lane * 8;
            const int ic = min(i, H - 8);
#pragma unroll
            for (int q = 0; q < kGuShMaxRows; ++q) {
                const int r = ra + min(q, nr - 1);
                b.w[q] = *reinterpret_cast<const u4 *>(p.sh_gate + (size_t)r * H + ic);
                b.w[kGuShMaxRows + q] = *reinterpret_cast<const u4 *>(p.sh_up + (size_t)r * H + ic);
            }
            b.x = *reinterpret_cast<const u4 *>(p.x + ic);
            if (i >= H) b.x = u4{0u, 0u, 0u, 0u};
        };
        auto compute = [&](const Slice &b) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float x0 = bf16f(b.x[h] & 0xffffu), x1 = bf16f(b.x[h] >> 16);
#pragma unroll
                for (int q = 0; q < 2 * kGuShMaxRows; ++q) {
                    acc[q] = fmaf(bf16f(b.w[q][h] & 0xffffu), x0, acc[q]);
                    acc[q] = fmaf(bf16f(b.w[q][h] >> 16), x1, acc[q]);
                }
            }
        };
        Slice b0, b1;
        load(0, b0);
        load(min(1, NS - 1), b1);
        for (int sl = 0; sl < NS; sl += 2) {
            compute(b0);
            load(min(sl + 2, NS - 1), b0);
            if (sl + 1 < NS) compute(b1);
            load(min(sl + 3, NS - 1), b1);
        }
#pragma unroll
        for (int q = 0; q < 2 * kGuShMaxRows; ++q)
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) acc[q] += __shfl_xor(acc[q], o);
        if (lane == 0)
#pragma unroll
            for (int q = 0; q < kGuShMaxRows; ++q)
                if (q < nr) p.ash[ra + q] = act_fn(acc[q], acc[kGuShMaxRows + q], p.act, p.b1, p.b2);
    }
}

// UNITS: routed waves per block (the other waves run shared rows), chosen
// so both kinds of wave move about the same bytes. P2: the routed input comes
// as bf16 hi and lo planes (a latent z); MFMA column c reads plane c & 1 and
// the two columns' sums are added at the end, so the second plane costs no
// extra MFMA.
template <bool WIDE, int UNITS, bool P2>
__global__ __launch_bounds__(64 * kGuDecWaves) void k_gateup_dec(GateUpParams p)
{
    constexpr int NP = P2 ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4, col = lane & 15;
    const int H = p.Kr, KS = H >> 7, SR = H >> 5, NCH = (KS + 3) >> 2;  // H: the routed input width
    const int SRP = SR + kScPad;
    const int RT = p.I / kGuUnitRows;
    const int nunits = p.K * RT;
    const int b = blockIdx.x;

    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *x_l = lds;                   // [NP][H]       the routed input, bf16
    uint8_t *sc_l = x_l + 2 * H * NP;     // [UNITS][2][16][H/32 + pad] unit scale rows

    // this wave's routed unit (waves 0..UNITS-1) and its expert
    const int u = UNITS * b + wave;
    const bool routed = wave < UNITS && u < nunits;
    const int slot = routed ? u / RT : 0, rt = routed ? u - (u / RT) * RT : 0;
    int e = routed ? p.idx[slot] : 0;
    const bool active = routed && e >= 0 && e < p.E;  // an invalid id: nothing (the combine counts it)
    e = active ? e : 0;
    const uint8_t *gpe = p.gp + e * p.g_sp, *upe = p.up + e * p.u_sp;
    const uint32_t po = ((uint32_t)rt * kGuUnitRows + (lane & 15)) * ((uint32_t)H >> 1) + grp * 16;

    struct Chunk {
        u4 a[4][2];  // [step][gate, up]
    };
    // unconditional loads (a step past K re-reads the last step; never used)
    auto load = [&](int c, Chunk &bf) {
        static_for<0, 4>([&](auto s_) {
            constexpr int st = decltype(s_)::value;
            const uint32_t k = (uint32_t)min(4 * c + st, KS - 1) * 64;
            bf.a[st][0] = *reinterpret_cast<const u4 *>(gpe + (po + k));
            bf.a[st][1] = *reinterpret_cast<const u4 *>(upe + (po + k));
        });
    };

    // Staging: all staging loads first, then the routed waves' first two
    // weight chunks, then the LDS stores (which wait only for the staging
    // loads). A unit's scale rows are 16 consecutive rows, contiguous.
    Chunk b0, b1;
    if constexpr (WIDE) {  // SR % 16 == 0
        const int nxq = (H >> 3) * NP;  // u4 count of the bf16 input planes
        const int nrow = SR >> 4, nsc = UNITS * 2 * kGuUnitRows * nrow;
        u4 tq[kGuStgQ], ts[kGuStgS];
#pragma unroll
        for (int q = 0; q < kGuStgQ; ++q) {
            const int i = min((int)threadIdx.x + q * 64 * kGuDecWaves, nxq - 1);
            const int pl = P2 ? i / (H >> 3) : 0, ii = i - pl * (H >> 3);
            tq[q] = *reinterpret_cast<const u4 *>((pl ? p.xr_lo : p.xr) + 8 * ii);
        }
#pragma unroll
        for (int q = 0; q < kGuStgS; ++q) {
            const int i = min((int)threadIdx.x + q * 64 * kGuDecWaves, nsc - 1);
            const int un = i / (2 * kGuUnitRows * nrow), rem = i - un * (2 * kGuUnitRows * nrow);
            const int mat = rem / (kGuUnitRows * nrow), rem2 = rem - mat * (kGuUnitRows * nrow);
            const int uu = min(UNITS * b + un, nunits - 1);
            const int su = uu / RT, srt = uu - su * RT;
            int se = p.idx[su];
            se = (se >= 0 && se < p.E) ? se : 0;
            const uint8_t *sbase = mat ? p.us + se * p.u_ss : p.gs + se * p.g_ss;
            ts[q] = *reinterpret_cast<const u4 *>(sbase + (size_t)srt * kGuUnitRows * SR + 16 * rem2);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
            load(0, b0);
            load(min(1, NCH - 1), b1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kGuStgQ; ++q) {
            const int i = (int)threadIdx.x + q * 64 * kGuDecWaves;
            if (i < nxq) *reinterpret_cast<u4 *>(x_l + 16 * i) = tq[q];
        }
#pragma unroll
        for (int q = 0; q < kGuStgS; ++q) {
            const int i = (int)threadIdx.x + q * 64 * kGuDecWaves;
            if (i < nsc) {
                const int row = i / nrow, o = i - row * nrow;  // row over [unit][mat][16]
                *reinterpret_cast<u4 *>(sc_l + row * SRP + 16 * o) = ts[q];
            }
        }
    } else {  // short rows (small layers): byte copies
        for (int i = threadIdx.x; i < H * NP; i += blockDim.x)
            reinterpret_cast<uint16_t *>(x_l)[i] = (P2 && i >= H) ? p.xr_lo[i - H] : p.xr[i];
        for (int i = threadIdx.x; i < UNITS * 2 * kGuUnitRows * SR; i += blockDim.x) {
            const int row = i / SR, o = i - row * SR;
            const int un = row / (2 * kGuUnitRows), mat = (row / kGuUnitRows) & 1, r = row % kGuUnitRows;
            const int uu = min(UNITS * b + un, nunits - 1);
            const int su = uu / RT, srt = uu - su * RT;
            int se = p.idx[su];
            se = (se >= 0 && se < p.E) ? se : 0;
            const uint8_t *sbase = mat ? p.us + se * p.u_ss : p.gs + se * p.g_ss;
            sc_l[row * SRP + o] = sbase[((size_t)srt * kGuUnitRows + r) * SR + o];
        }
        if (active) {
            load(0, b0);
            load(min(1, NCH - 1), b1);
        }
    }
    __syncthreads();

    if (wave >= UNITS) {  // the shared expert's slice of rows, split over the shared waves
        if (p.Is > 0) {
            const int64_t ns = (int64_t)gridDim.x * (kGuDecWaves - UNITS), si = (int64_t)b * (kGuDecWaves - UNITS) + (wave - UNITS);
            shared_gateup_rows(p, (int)(p.Is * si / ns), (int)(p.Is * (si + 1) / ns));
        }
        return;
    }
    if (!active) return;

    // B operand: the bf16 token, the same in every column (columns 1..15 are
    // copies). Lane group grp's 16-byte weight load of 128-K step k holds
    // K = 128k + 32 grp + [0, 32); MFMA sub-step ss takes K = 128k + 32 grp +
    // 8 ss + [0, 8) on both sides.
    const uint8_t *xb = x_l + (P2 ? (col & 1) * 2 * H : 0) + 64 * grp;  // P2: column c reads plane c & 1
    const uint8_t *s_g = sc_l + (wave * 2 * kGuUnitRows + (lane & 15)) * SRP;  // this lane's gate row
    const uint8_t *s_u = s_g + kGuUnitRows * SRP;
    v4f accg = v4f{0.0f, 0.0f, 0.0f, 0.0f}, accu = accg;
    auto compute = [&](int c, const Chunk &bf) {
        uint32_t sg, su;
        if constexpr (WIDE) {
            sg = gather_scales(*reinterpret_cast<const u4 *>(s_g + 16 * c), grp);
            su = gather_scales(*reinterpret_cast<const u4 *>(s_u + 16 * c), grp);
        } else {  // short rows: steps past K are never multiplied
            sg = su = 0x7f7f7f7fu;
            for (int st = 0; st < 4 && 4 * c + st < KS; ++st) {
                const int o = (4 * c + st) * 4 + grp, sh8 = 8 * st;
                const uint32_t m = ~(0xffu << sh8);
                sg = (sg & m) | ((uint32_t)s_g[o] << sh8);
                su = (su & m) | ((uint32_t)s_u[o] << sh8);
            }
        }
        static_for<0, 4>([&](auto s_) {
            constexpr int st = decltype(s_)::value;
            if (4 * c + st < KS) {
                const uint32_t k = 4 * c + st;
                const float fg = e8m0_to_f32((sg >> (8 * st)) & 0xffu), fu = e8m0_to_f32((su >> (8 * st)) & 0xffu);
#pragma unroll
                for (int ss = 0; ss < 4; ++ss) {
                    const bf8 B = as_bf8(*reinterpret_cast<const u4 *>(xb + k * 256 + 16 * ss));
                    accg = mfma_bf16(dequant8_bf16(bf.a[st][0][ss], fg), B, accg);
                    accu = mfma_bf16(dequant8_bf16(bf.a[st][1][ss], fu), B, accu);
                }
            }
        });
    };
    for (int c = 0; c < NCH; c += 2) {
        compute(c, b0);
        load(min(c + 2, NCH - 1), b0);
        if (c + 1 < NCH) compute(c + 1, b1);
        load(min(c + 3, NCH - 1), b1);
    }

    // every column holds the token's result (P2: columns 0 and 1 its hi and
    // lo parts, added here): lane 16g (column 0) has rows 4g..4g+3
    if constexpr (P2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            accg[r] += __shfl_xor(accg[r], 1);
            accu[r] += __shfl_xor(accu[r], 1);
        }
    }
    if (col == 0) {
        float4 a4;
        a4.x = act_fn(accg[0], accu[0], p.act, p.b1, p.b2);
        a4.y = act_fn(accg[1], accu[1], p.act, p.b1, p.b2);
        a4.z = act_fn(accg[2], accu[2], p.act, p.b1, p.b2);
        a4.w = act_fn(accg[3], accu[3], p.act, p.b1, p.b2);
        *reinterpret_cast<float4 *>(p.act_f + (size_t)slot * p.I + rt * kGuUnitRows + 4 * grp) = a4;
    }
}

// Down projection, T = 1. Block (j, i) of K x M blocks takes router slot j,
// the 16-row tiles [T16*i/M, T16*(i+1)/M) of H (T16 = H/16) and the shared
// rows [H*(jM+i)/(KM), ...): every block moves about the same bytes. The
// slot's fp32 activation is expanded into 4 e4m3 terms (one E8M0 scale per
// 32 elements per term; 8 lanes per 32-element block, DPP maxima) while it
// is staged in LDS, with the tiles' E8M0 rows; wave w takes tiles t0+w,
// t0+w+4, ... (K in chunks of 4 MFMA steps, a
// 4-deep register ring) and shared rows r0+w, r0+w+4, ... (bf16, fp32 FMA,
// loads issued before the routed stream). Results go to the staging rows
// ys[j][.] and ys[k][.] (shared); the combine sums them in router order.
struct DownDecParams {
    const uint8_t *dp, *ds;
    int64_t d_sp, d_ss;
    int H, I, E, K, Is, M;
    int Hr;     // routed output rows (H, or the latent)
    float *ysh; // the shared expert's rows fp32 [H], or null: ys slot k
    const int32_t *idx;
    const float *act_f;  // fp32 activations [k][I]
    const uint16_t *sh_down;
    const float *ash;
    float *ys;
};

constexpr int kDnDecWaves = 4;
constexpr int kDnMaxTiles = 16;      // tiles per block (LDS sizing)
constexpr int kDnShPerWave = 4;      // shared rows per wave (at most)
constexpr int kDnShSl = 3;           // shared slices of 512 per load group (the first prefetched)
constexpr int kDnStgQ = 3;           // activation float4s per thread (I <= 3072)
constexpr int kDnStgS = 4;           // scale-row staging copies per thread

__host__ __device__ constexpr int dn_dec_lds_bytes(int I)
{
    return 4 * (I + kXqPad) + 4 * (I / 32) + 16 * kDnMaxTiles * (I / 32 + kScPad) + 4 * 16 * kDnMaxTiles +
           4 * 16;
}

template <bool WIDE>
__global__ __launch_bounds__(64 * kDnDecWaves) void k_down_dec(DownDecParams p)
{
    static_assert(kATerms == 4, "4-term expansion");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4, col = lane & 15;
    const int I = p.I, KS = I >> 7, SR = I >> 5, NCH = (KS + 3) >> 2;
    const int AQS = I + kXqPad, SRP = SR + kScPad;
    const int T16 = p.Hr >> 4, M = p.M;
    const int j = blockIdx.x / M, i = blockIdx.x - j * M;
    const int t0 = T16 * i / M, t1 = T16 * (i + 1) / M, nt = t1 - t0;
    const int nblk = p.K * M;
    const int r0 = (int)((int64_t)p.H * blockIdx.x / nblk), r1 = (int)((int64_t)p.H * (blockIdx.x + 1) / nblk);
    const int e_raw = p.idx[j];
    const bool ok = e_raw >= 0 && e_raw < p.E;  // an invalid id: zeros (the combine counts it)
    const int e = ok ? e_raw : 0;

    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *aq_l = lds;                                   // [4][I + pad] activation terms of slot j
    uint8_t *as_l = aq_l + 4 * AQS;                        // [4][I/32]    their scales
    uint8_t *sc_l = as_l + 4 * SR;                         // [nt*16][I/32 + pad] the tiles' scale rows
    float *y_l = reinterpret_cast<float *>(sc_l + 16 * kDnMaxTiles * SRP);  // [nt*16]
    float *sh_l = y_l + 16 * kDnMaxTiles;                                   // [r1 - r0]

    const uint8_t *ape = p.dp + (int64_t)e * p.d_sp;
    const uint8_t *ase = p.ds + (int64_t)e * p.d_ss + (size_t)t0 * 16 * SR;
    const float *afj = p.act_f + (size_t)j * I;
    const int ntw = (nt - wave + kDnDecWaves - 1) / kDnDecWaves;  // tiles of this wave
    const int nq = ok ? ntw * NCH : 0;                            // chunks of this wave
    const uint32_t rowb = (uint32_t)I >> 1;
    const uint32_t pl = (uint32_t)(lane & 15) * rowb + grp * 16;

    // shared rows of this wave (prefetched) and the shared activation
    const int nsr = (r1 - r0 - wave + kDnDecWaves - 1) / kDnDecWaves;
    const int Is = p.Is;
    u4 shw[kDnShPerWave][kDnShSl];
    float4 shx[kDnShSl][2];
    const bool sh_pf = Is > 0 && nsr <= kDnShPerWave;  // the first kDnShSl slices of the shared rows
    if (sh_pf) {
#pragma unroll
        for (int c = 0; c < kDnShSl; ++c) {
            const int ic = min(c * 512 + lane * 8, Is - 8);
#pragma unroll
            for (int q = 0; q < kDnShPerWave; ++q) {
                const int r = r0 + wave + kDnDecWaves * min(q, max(nsr - 1, 0));
                shw[q][c] = *reinterpret_cast<const u4 *>(p.sh_down + (size_t)min(r, p.H - 1) * Is + ic);
            }
            shx[c][0] = *reinterpret_cast<const float4 *>(p.ash + ic);
            shx[c][1] = *reinterpret_cast<const float4 *>(p.ash + ic + 4);
        }
    }

    struct Chunk {
        u4 a[4];
    };
    auto load = [&](int q, Chunk &bf) {
        const int tw = q / NCH, c = q - tw * NCH;
        const uint32_t tile = (uint32_t)(t0 + wave + kDnDecWaves * tw);
        const uint32_t base = tile * 16u * rowb + pl;
        static_for<0, 4>([&](auto s_) {
            constexpr int st = decltype(s_)::value;
            const uint32_t k = (uint32_t)min(4 * c + st, KS - 1);
            bf.a[st] = *reinterpret_cast<const u4 *>(ape + (base + k * 64));
        });
    };

    // staging loads (the slot's activation, the tiles' scale rows), then the
    // first 4 weight chunks, then the expansion and the LDS stores
    Chunk b0, b1, b2, b3;
    float4 av[kDnStgQ];  // elements 4 (tid + 256 q) + [0, 4)
#pragma unroll
    for (int q = 0; q < kDnStgQ; ++q)
        av[q] = *reinterpret_cast<const float4 *>(afj + min(4 * ((int)threadIdx.x + q * 64 * kDnDecWaves), I - 4));
    if constexpr (WIDE) {  // SR % 16 == 0
        const int nrow = SR >> 4, nsc = nt * 16 * nrow;
        u4 ts[kDnStgS];
#pragma unroll
        for (int q = 0; q < kDnStgS; ++q) {
            const int ii = min((int)threadIdx.x + q * 64 * kDnDecWaves, nsc - 1);
            ts[q] = *reinterpret_cast<const u4 *>(ase + 16 * ii);  // the tiles' rows are contiguous
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nq > 0) {
            load(0, b0);
            load(min(1, nq - 1), b1);
            load(min(2, nq - 1), b2);
            load(min(3, nq - 1), b3);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kDnStgS; ++q) {
            const int ii = (int)threadIdx.x + q * 64 * kDnDecWaves;
            if (ii < nsc) {
                const int row = ii / nrow, o = ii - row * nrow;
                *reinterpret_cast<u4 *>(sc_l + row * SRP + 16 * o) = ts[q];
            }
        }
    } else {  // short rows (small layers): byte copies
        for (int ii = threadIdx.x; ii < nt * 16 * SR; ii += blockDim.x) {
            const int row = ii / SR, o = ii - row * SR;
            sc_l[row * SRP + o] = ase[ii];
        }
        if (nq > 0) {
            load(0, b0);
            load(min(1, nq - 1), b1);
            load(min(2, nq - 1), b2);
            load(min(3, nq - 1), b3);
        }
    }
    // activation -> 4 e4m3 terms; the octet of lanes 8m..8m+7 holds one
    // 32-element block (I is a multiple of 128: whole octets), every lane
    // splits (clamped copies past I are not stored)
#pragma unroll
    for (int q = 0; q < kDnStgQ; ++q) {
        const int i4 = 4 * ((int)threadIdx.x + q * 64 * kDnDecWaves);
        if (q * 4 * 64 * kDnDecWaves < I) {
            uint32_t code4[kATerms];
            int sbt[kATerms];
            split_e4m3_octet<kATerms>(av[q], code4, sbt);
            if (i4 < I)
#pragma unroll
                for (int k = 0; k < kATerms; ++k) {
                    *reinterpret_cast<uint32_t *>(aq_l + k * AQS + i4) = code4[k];
                    if ((i4 & 31) == 0) as_l[k * SR + (i4 >> 5)] = (uint8_t)sbt[k];
                }
        }
    }
    __syncthreads();

    const int term = col & 3;  // columns 4..15: copies of columns 0..3, ignored
    const uint8_t *bb = aq_l + term * AQS + grp * 16;
    const uint8_t *bsr = as_l + term * SR;
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // chunk q: tile t0 + wave + 4*(q / NCH), steps 4*(q % NCH)..+3; a tile's
    // result is parked in LDS when its last chunk is done (no global stores
    // inside the loop, so the weight loads' wait counts stay exact)
    auto compute = [&](int q, const Chunk &bf) {
        if (q >= nq) return;
        const int tw = q / NCH, c = q - tw * NCH;
        const int trow = (wave + kDnDecWaves * tw) * 16;  // first row of the tile, block-relative
        const uint8_t *sr = sc_l + (trow + (lane & 15)) * SRP;
        uint32_t sa, sb;
        if constexpr (WIDE) {
            sa = gather_scales(*reinterpret_cast<const u4 *>(sr + 16 * c), grp);
            sb = gather_scales(*reinterpret_cast<const u4 *>(bsr + 16 * c), grp);
        } else {  // short rows: steps past K left at 127 (never multiplied)
            sa = sb = 0x7f7f7f7fu;
            for (int st = 0; st < 4 && 4 * c + st < KS; ++st) {
                const int o = (4 * c + st) * 4 + grp, sh8 = 8 * st;
                const uint32_t m = ~(0xffu << sh8);
                sa = (sa & m) | ((uint32_t)sr[o] << sh8);
                sb = (sb & m) | ((uint32_t)bsr[o] << sh8);
            }
        }
        const uint32_t drop = ff_bytes(sa);  // scale byte 255: the group drops out
        sa ^= drop;
        static_for<0, 4>([&](auto s_) {
            constexpr int st = decltype(s_)::value;
            if (4 * c + st < KS) {
                const uint32_t k = 4 * c + st;
                const v8i B = b_operand(*reinterpret_cast<const u4 *>(bb + k * 128),
                                        *reinterpret_cast<const u4 *>(bb + k * 128 + 64));
                const u4 av = ((drop >> (8 * st + 7)) & 1u) ? u4{0u, 0u, 0u, 0u} : bf.a[st];
                acc = mfma_fp4_fp8<st>(a_operand(av), B, acc, (int)sa, (int)sb);
            }
        });
        if (c == NCH - 1) {
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                y[r] = acc[r] + __shfl_xor(acc[r], 1);
                y[r] += __shfl_xor(y[r], 2);
            }
            if (col == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) y_l[trow + 4 * grp + r] = y[r];
            acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    for (int q = 0; q < nq; q += 4) {
        compute(q, b0);
        load(min(q + 4, nq - 1), b0);
        compute(q + 1, b1);
        load(min(q + 5, nq - 1), b1);
        compute(q + 2, b2);
        load(min(q + 6, nq - 1), b2);
        compute(q + 3, b3);
        load(min(q + 7, nq - 1), b3);
    }

    // shared rows r0 + wave + 4q
    if (Is > 0) {
        auto dot8 = [&](float &a, const u4 &w4, const float4 &x0, const float4 &x1) {
            float v = a;
            v = fmaf(bf16f(w4[0] & 0xffffu), x0.x, v);
            v = fmaf(bf16f(w4[0] >> 16), x0.y, v);
            v = fmaf(bf16f(w4[1] & 0xffffu), x0.z, v);
            v = fmaf(bf16f(w4[1] >> 16), x0.w, v);
            v = fmaf(bf16f(w4[2] & 0xffffu), x1.x, v);
            v = fmaf(bf16f(w4[2] >> 16), x1.y, v);
            v = fmaf(bf16f(w4[3] & 0xffffu), x1.z, v);
            v = fmaf(bf16f(w4[3] >> 16), x1.w, v);
            a = v;
        };
        if (sh_pf) {  // slices of 512 in groups of kDnShSl, all the wave's rows at once
            float a4[kDnShPerWave];
#pragma unroll
            for (int q = 0; q < kDnShPerWave; ++q) a4[q] = 0.0f;
            for (int c0 = 0; c0 < Is; c0 += 512 * kDnShSl) {
                if (c0 > 0) {  // the first group was loaded before the routed stream
#pragma unroll
                    for (int c = 0; c < kDnShSl; ++c) {
                        const int ic = min(c0 + c * 512 + lane * 8, Is - 8);
#pragma unroll
                        for (int q = 0; q < kDnShPerWave; ++q) {
                            const int r = r0 + wave + kDnDecWaves * min(q, max(nsr - 1, 0));
                            shw[q][c] = *reinterpret_cast<const u4 *>(p.sh_down + (size_t)min(r, p.H - 1) * Is + ic);
                        }
                        shx[c][0] = *reinterpret_cast<const float4 *>(p.ash + ic);
                        shx[c][1] = *reinterpret_cast<const float4 *>(p.ash + ic + 4);
                    }
                }
#pragma unroll
                for (int c = 0; c < kDnShSl; ++c)
                    if (c0 + c * 512 + lane * 8 < Is)
#pragma unroll
                        for (int q = 0; q < kDnShPerWave; ++q) dot8(a4[q], shw[q][c], shx[c][0], shx[c][1]);
            }
#pragma unroll
            for (int q = 0; q < kDnShPerWave; ++q) {
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) a4[q] += __shfl_xor(a4[q], o);
                if (lane == 0 && q < nsr) sh_l[wave + kDnDecWaves * q] = a4[q];
            }
        } else {
            for (int q = 0; q < nsr; ++q) {
                const int r = r0 + wave + kDnDecWaves * q;
                float a = 0.0f;
                for (int ii = lane * 8; ii < Is; ii += 512) {
                    const float4 x0 = *reinterpret_cast<const float4 *>(p.ash + ii);
                    const float4 x1 = *reinterpret_cast<const float4 *>(p.ash + ii + 4);
                    dot8(a, *reinterpret_cast<const u4 *>(p.sh_down + (size_t)r * Is + ii), x0, x1);
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o);
                if (lane == 0) sh_l[wave + kDnDecWaves * q] = a;
            }
        }
    }
    __syncthreads();
    for (int ii = threadIdx.x; ii < nt * 16; ii += blockDim.x)
        p.ys[(size_t)j * p.Hr + (size_t)t0 * 16 + ii] = ok ? y_l[ii] : 0.0f;
    if (Is > 0) {
        float *yshr = p.ysh ? p.ysh : p.ys + (size_t)p.K * p.Hr;
        for (int ii = threadIdx.x; ii < r1 - r0; ii += blockDim.x) yshr[r0 + ii] = sh_l[ii];
    }
}

// Router-order combine: out[t][o] = sum_j w[t][j] * ys[t][j][o] (j = 0..k-1
// in order, one fma each), then + ys[t][k][o] (the shared expert, if any).
// A slot with an out-of-range id adds nothing (its staging row is loaded but
// dropped) and is counted once here. A thread takes 4 consecutive outputs
// (16-byte loads); the loads of up to 16 slots are issued before the first fma.
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void k_combine(const float *__restrict__ ys,
                                                             const float *__restrict__ w,
                                                             const int32_t *__restrict__ idx, int T, int K,
                                                             int H, int E, int shared, float *__restrict__ out,
                                                             unsigned long long *errors, int resid,
                                                             uint16_t *__restrict__ ob)
{
    const int64_t i4 = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;  // float4 index
    const int H4 = H >> 2;
    if (i4 < (int64_t)T * H4) {
        const int64_t t = i4 / H4;
        const int o = (int)(i4 - t * H4) * 4;
        const float *y = ys + (size_t)t * (K + 1) * H + o;
        const float *wt = w + (size_t)t * K;
        const int32_t *it = idx + (size_t)t * K;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int j0 = 0; j0 < K; j0 += 16) {
            // ids, weights and staging rows are loaded together (clamped,
            // unconditional); a slot with an invalid id is dropped after
            float4 v[16];
            float wj[16];
            int e[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int j = min(j0 + q, K - 1);
                e[q] = it[j];
                wj[q] = wt[j];
                v[q] = *reinterpret_cast<const float4 *>(y + (size_t)j * H);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (j0 + q < K && e[q] >= 0 && e[q] < E) {
                    acc.x = fmaf(wj[q], v[q].x, acc.x);
                    acc.y = fmaf(wj[q], v[q].y, acc.y);
                    acc.z = fmaf(wj[q], v[q].z, acc.z);
                    acc.w = fmaf(wj[q], v[q].w, acc.w);
                }
            }
        }
        if (shared) {
            const float4 sv = *reinterpret_cast<const float4 *>(y + (size_t)K * H);
            acc.x += sv.x;
            acc.y += sv.y;
            acc.z += sv.z;
            acc.w += sv.w;
        }
        float4 *op = reinterpret_cast<float4 *>(out + (size_t)t * H + o);
        if (resid) {  // the residual stream: h + (complete layer output)
            const float4 hv = *op;
            acc = make_float4(hv.x + acc.x, hv.y + acc.y, hv.z + acc.z, hv.w + acc.w);
        }
        *op = acc;
        if (ob)
            *reinterpret_cast<uint2 *>(ob + (size_t)t * H + o) =
                make_uint2(bf16_rne_u32(acc.x) | (bf16_rne_u32(acc.y) << 16),
                           bf16_rne_u32(acc.z) | (bf16_rne_u32(acc.w) << 16));
    }
    // ids outside [0, E), counted once each, spread over the grid (one
    // assignment per thread: the grid has T H/4 >= T K threads; a loop in one
    // block would hold the kernel's end by a cache round trip per iteration)
    for (int64_t a = i4; a < (int64_t)T * K; a += (int64_t)gridDim.x * kCombineThreads)
        if (idx[a] < 0 || idx[a] >= E) atomicAdd(errors, 1ull);
}

}  // namespace

// Tokens per batched-router block: 128 from 128 tokens on, else 64.
static int router_wt(int64_t T) { return T >= 128 ? 4 : 2; }

// Hidden-dimension slices of the batched router: about one block per block
// slot of the chip (256 CUs; a CU holds one 1024-thread block or two
// 512-thread ones), slices of at least 256 elements (whole 64-element
// stages).
int router_splits(int64_t T, int E, int H)
{
    const int64_t wt = router_wt(T), slots = wt == 4 ? 256 : 512;
    const int64_t tiles = (int64_t)((E + kRtE - 1) / kRtE) * ((T + 32 * wt - 1) / (32 * wt));
    const int64_t want = (slots + tiles / 2) / tiles;
    const int64_t S = std::max<int64_t>(1, std::min<int64_t>(want, H / 256));
    return (int)((H + router_kspan(H, (int)S) - 1) / router_kspan(H, (int)S));
}

int router_kspan(int H, int S) { return (H / kRtK + S - 1) / S * kRtK; }

static bool set_router_lds()
{
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_router_mm<2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, rt_lds_bytes<2>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_router_mm<4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, rt_lds_bytes<4>());
    return true;
}

template <int NQ>
static void topk_launch(int T, hipStream_t s, const float *sc, const float *ch, const LayerView &L,
                        int32_t *idx, float *w)
{
    // 16-byte loads need whole quads of experts per lane and 16-byte aligned
    // rows (the workspace regions are 256-aligned)
    if (NQ % 4 == 0 && L.E % 4 == 0)
        k_topk<NQ, (NQ % 4 == 0)><<<T, 64, 0, s>>>(sc, ch, L.E, L.K, L.renorm, L.routed_scale, idx, w);
    else
        k_topk<NQ, false><<<T, 64, 0, s>>>(sc, ch, L.E, L.K, L.renorm, L.routed_scale, idx, w);
}

hipError_t launch_route(const LayerView &L, const uint16_t *x, int T, int32_t *idx, float *w,
                        float *logits, char *ws, const WsLayout &lay, hipStream_t s, Profiler *prof)
{
    float *sc = reinterpret_cast<float *>(ws + lay.sc);
    float *ch = reinterpret_cast<float *>(ws + lay.ch);
    {
        StageMark m(prof, K3MOE_STAGE_ROUTER, s);
        if (T <= kRouterWaveMaxT) {
            if (T == 1)
                k_router<true><<<dim3((L.E + 3) / 4, 1), 256, 0, s>>>(x, L.router_w, L.router_bias, L.H, L.E,
                                                                      sc, ch, logits);
            else
                k_router<false><<<dim3((L.E + 3) / 4, T), 256, 0, s>>>(x, L.router_w, L.router_bias, L.H, L.E,
                                                                       sc, ch, logits);
        } else {
            static const bool lds_set = set_router_lds();  // once per process (thread-safe static)
            (void)lds_set;
            const int S = router_splits(T, L.E, L.H);
            const int kspan = router_kspan(L.H, S);
            double *part = S > 1 ? reinterpret_cast<double *>(ws + lay.rt_part) : nullptr;
            const int WT = router_wt(T);
            const dim3 grid((L.E + kRtE - 1) / kRtE, (unsigned)((T + 32 * WT - 1) / (32 * WT)), S);
            if (WT == 4)
                k_router_mm<4><<<grid, 1024, rt_lds_bytes<4>(), s>>>(x, L.router_w, T, L.H, L.E, kspan, part,
                                                                      L.router_bias, sc, ch, logits);
            else
                k_router_mm<2><<<grid, 512, rt_lds_bytes<2>(), s>>>(x, L.router_w, T, L.H, L.E, kspan, part,
                                                                     L.router_bias, sc, ch, logits);
            if (S > 1) {
                const int64_t n = (int64_t)T * L.E;
                k_router_reduce<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, S, T, L.E, L.router_bias, sc,
                                                                            ch, logits);
            }
        }
    }
    {
        StageMark m(prof, K3MOE_STAGE_TOPK, s);
        (void)launch_topk(L, T, sc, ch, idx, w, s);
    }
    return hipGetLastError();
}

// The router rows of one token (one wave per expert): scores and selection
// scores into sc, ch; fp32 logits when asked.
hipError_t launch_router_t1(const LayerView &L, const uint16_t *x, float *sc, float *ch, float *logits,
                            hipStream_t s)
{
    k_router<true><<<dim3((L.E + 3) / 4, 1), 256, 0, s>>>(x, L.router_w, L.router_bias, L.H, L.E, sc, ch,
                                                          logits);
    return hipGetLastError();
}

hipError_t launch_topk(const LayerView &L, int T, const float *sc, const float *ch, int32_t *idx, float *w,
                       hipStream_t s)
{
    const int nq = (L.E + 63) / 64;
    if (nq <= 1) topk_launch<1>(T, s, sc, ch, L, idx, w);
    else if (nq <= 2) topk_launch<2>(T, s, sc, ch, L, idx, w);
    else if (nq <= 4) topk_launch<4>(T, s, sc, ch, L, idx, w);
    else if (nq <= 8) topk_launch<8>(T, s, sc, ch, L, idx, w);
    else if (nq <= 16) topk_launch<16>(T, s, sc, ch, L, idx, w);
    else if (nq <= 32) topk_launch<32>(T, s, sc, ch, L, idx, w);
    else topk_launch<64>(T, s, sc, ch, L, idx, w);
    return hipGetLastError();
}

// Sizes the single-token kernels take (one pass of LDS staging copies per
// thread; row tiles dividing I and H; a down block's tiles fit its LDS).
static int down_blocks_per_slot(const LayerView &L, int ncu)
{
    const int T16 = L.EK / 16;  // routed output tiles
    int M = std::max(1, (2 * ncu + L.K - 1) / L.K);
    M = std::min(M, T16);
    // tiles per block fit the LDS staging, and their scale rows one pass of
    // the staging copies (wide rows)
    auto fits = [&](int m) {
        const int nt = (T16 + m - 1) / m;
        return nt <= kDnMaxTiles && (L.I % 512 != 0 || nt * 16 * (L.I / 512) <= 64 * kDnDecWaves * kDnStgS);
    };
    while (M < T16 && !fits(M)) ++M;
    return M;
}

// Routed waves per gate/up block: both kinds of wave should move about the
// same bytes (a routed unit: 16 rows of gate and up; the shared rows shared
// out over the other waves of every block).
static int gu_dec_units(const LayerView &L)
{
    const double routed = (double)L.K * L.I * L.EK * 2 * (0.5 + 1.0 / 32), shared = (double)L.Is * L.H * 4;
    const int u = (int)(4.0 * routed / (routed + shared) + 0.5);
    return u <= 2 ? 2 : 3;
}

static bool decode_path_ok(const LayerView &L)
{
    // a latent layer: whole 512-groups (the two-plane staging takes the wide form)
    if (L.Lt > 0 && (L.EK % 512 != 0 || L.H % 512 != 0)) return false;
    const int np = L.Lt > 0 ? 2 : 1;
    const bool gu = L.EK % 512 != 0 || np * L.EK / 8 <= 64 * kGuDecWaves * kGuStgQ;
    const bool gu_sc = L.EK % 512 != 0 || kGuDecMaxUnits * 2 * kGuUnitRows * (L.EK / 512) <= 64 * kGuDecWaves * kGuStgS;
    // the activation staging; one tile's scale rows per staging pass at least
    // (down_blocks_per_slot takes enough blocks for the rest)
    const bool dn = L.I <= 4 * 64 * kDnDecWaves * kDnStgQ &&
                    (L.I % 512 != 0 || 16 * (L.I / 512) <= 64 * kDnDecWaves * kDnStgS);
    return gu && gu_sc && dn && L.I % kGuUnitRows == 0 && L.EK % 16 == 0 && L.EK >= 16 * kDnDecWaves &&
           L.H >= 16 * kDnDecWaves;
}

// T = 1: token fp8 expansion, gate/up, down, router-order combine. The
// router slots are the assignment list (no permutation).
// xr, xr_lo: the routed input (x, or a latent z as hi and lo planes); ysh:
// the shared rows' own buffer (latent) or null (slot k of the staging rows);
// out null: no combine (the latent layer combines at its own width).
static hipError_t launch_forward_t1(const LayerView &L, const uint16_t *x, const uint16_t *xr,
                                    const uint16_t *xr_lo, const int32_t *idx, const float *w, float *out,
                                    float *act, float *ash, char *ys_base, float *ysh, hipStream_t s,
                                    Profiler *prof, const OutEpi &epi)
{
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    GateUpParams gp{};
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
    gp.E = L.E;
    gp.act = L.act;
    gp.Is = L.Is;
    gp.b1 = L.b1;
    gp.b2 = L.b2;
    gp.x = x;
    gp.xr = xr;
    gp.xr_lo = xr_lo;
    gp.Kr = L.EK;
    gp.idx = idx;
    gp.act_f = act;
    gp.sh_gate = L.sh_gate;
    gp.sh_up = L.sh_up;
    gp.ash = ash;
    {
        StageMark m(prof, K3MOE_STAGE_GATEUP, s);
        const int nunits = L.K * (L.I / kGuUnitRows), units = gu_dec_units(L);
        const unsigned nblk = (unsigned)((nunits + units - 1) / units);
        const size_t lds = gu_dec_lds_bytes(L.EK, xr_lo ? 2 : 1);
        if (xr_lo)  // two planes: the wide form only (decode_path_ok)
            k_gateup_dec<true, 2, true><<<nblk, 64 * kGuDecWaves, lds, s>>>(gp);
        else if (L.EK % 512 == 0 && units == 2)
            k_gateup_dec<true, 2, false><<<nblk, 64 * kGuDecWaves, lds, s>>>(gp);
        else if (L.EK % 512 == 0)
            k_gateup_dec<true, 3, false><<<nblk, 64 * kGuDecWaves, lds, s>>>(gp);
        else if (units == 2)
            k_gateup_dec<false, 2, false><<<nblk, 64 * kGuDecWaves, lds, s>>>(gp);
        else
            k_gateup_dec<false, 3, false><<<nblk, 64 * kGuDecWaves, lds, s>>>(gp);
    }
    float *ys = reinterpret_cast<float *>(ys_base);
    DownDecParams dp{};
    dp.dp = L.dp;
    dp.ds = L.ds;
    dp.d_sp = L.d_sp;
    dp.d_ss = L.d_ss;
    dp.H = L.H;
    dp.Hr = L.EK;
    dp.ysh = ysh;
    dp.I = L.I;
    dp.E = L.E;
    dp.K = L.K;
    dp.Is = L.Is;
    dp.M = down_blocks_per_slot(L, ncu);
    dp.idx = idx;
    dp.act_f = gp.act_f;
    dp.sh_down = L.sh_down;
    dp.ash = ash;
    dp.ys = ys;
    {
        StageMark m(prof, K3MOE_STAGE_DOWN, s);
        const unsigned nblk = (unsigned)(L.K * dp.M);
        const size_t lds = dn_dec_lds_bytes(L.I) + 4 * (L.H / nblk + 1);  // + the block's shared rows
        if (L.I % 512 == 0)
            k_down_dec<true><<<nblk, 64 * kDnDecWaves, lds, s>>>(dp);
        else
            k_down_dec<false><<<nblk, 64 * kDnDecWaves, lds, s>>>(dp);
    }
    if (out) {
        StageMark m(prof, K3MOE_STAGE_COMBINE, s);
        k_combine<<<(unsigned)((L.H / 4 + kCombineThreads - 1) / kCombineThreads), kCombineThreads, 0, s>>>(
            ys, w, idx, 1, L.K, L.H, L.E, L.Is > 0, out, L.errors, epi.resid, epi.ob);
    }
    return hipGetLastError();
}

// One token of a latent layer on the single-token kernels: the routed
// experts read z's planes and write their rows (width EK) to the staging
// rows, the shared expert reads x and writes ysh [H].
hipError_t launch_latent_t1(const LayerView &L, const uint16_t *x, const uint16_t *zh, const uint16_t *zl,
                            const int32_t *idx, float *act, float *ash, char *ys_base, float *ysh, hipStream_t s,
                            Profiler *prof)
{
    return launch_forward_t1(L, x, zh, zl, idx, nullptr, nullptr, act, ash, ys_base, ysh, s, prof, OutEpi());
}

bool latent_t1_ok(const LayerView &L) { return decode_path_ok(L); }

// T > 1 (or shapes the single-token kernels do not take): token -> expert
// permutation, grouped GEMMs, router-order combine.
void launch_perm(const LayerView &L, const int32_t *idx, int T, char *ws, const WsLayout &lay, hipStream_t s,
                 Profiler *prof)
{
    int32_t *active_n = reinterpret_cast<int32_t *>(ws + lay.active_n);
    int32_t *active_e = reinterpret_cast<int32_t *>(ws + lay.active_e);
    int32_t *active_off = reinterpret_cast<int32_t *>(ws + lay.active_off);
    int32_t *sorted = reinterpret_cast<int32_t *>(ws + lay.sorted);
    const int nchunks = (T + kPermChunk - 1) / kPermChunk;
    StageMark m(prof, K3MOE_STAGE_PERM, s);
    if (nchunks == 1) {
        k_perm_small<<<1, 256, 0, s>>>(idx, T, L.K, L.E, active_n, active_e, active_off, sorted);
    } else {
        int32_t *chunk_cnt = reinterpret_cast<int32_t *>(ws + lay.chunk_cnt);
        k_perm_hist<<<nchunks, 256, 0, s>>>(idx, T, L.K, L.E, chunk_cnt);
        k_perm_scan<<<1, 1024, 0, s>>>(nchunks, L.E, chunk_cnt, active_n, active_e, active_off);
        k_perm_scatter<<<nchunks, 64, 0, s>>>(idx, T, L.K, L.E, chunk_cnt, sorted);
    }
}

// out[t][0..width) = router-order sum of the staging rows ys[t][j] (stride
// width, k + 1 slots), plus slot k when `shared`.
void launch_combine(const LayerView &L, const float *ys, const float *w, const int32_t *idx, int T, int width,
                    bool shared, float *out, hipStream_t s, const OutEpi &epi)
{
    const int64_t n4 = (int64_t)T * width / 4;
    k_combine<<<(unsigned)((n4 + kCombineThreads - 1) / kCombineThreads), kCombineThreads, 0, s>>>(
        ys, w, idx, T, L.K, width, L.E, shared, out, L.errors, epi.resid, epi.ob);
}

// Batches up to these sizes run one-token kernels once per token instead of
// one weight-streaming pass over the union of their experts. With the fused
// one-token kernels (full flat shape, a decoder-layer step of distinct
// routes per token) the per-token loop costs ~63 us a token and wins up to
// 8 tokens: T = 2 139 us against 166 for the older one-token kernels and a
// combine, T = 4 263 against 311, T = 5 322 against 357 streamed, T = 6 383
// against 415, T = 8 503 against 533. A batch whose tokens share most of
// their experts would stream faster, but the routes are on the device when
// this is decided. Shapes the fused kernels do not take use the older
// one-token kernels up to 4 tokens (T = 4 310 us against 354 streamed).
constexpr int kT1LoopMax = 4;
constexpr int kFusedLoopMax = 8;

hipError_t launch_forward(const LayerView &L, const uint16_t *x, int T, const int32_t *idx,
                          const float *w, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                          Profiler *prof, const OutEpi &epi)
{
    if (L.Lt > 0) return launch_latent_forward(L, x, T, idx, w, out, ws, lay, s, prof, epi);
    int32_t *active_n = reinterpret_cast<int32_t *>(ws + lay.active_n);
    int32_t *active_e = reinterpret_cast<int32_t *>(ws + lay.active_e);
    int32_t *active_off = reinterpret_cast<int32_t *>(ws + lay.active_off);
    int32_t *sorted = reinterpret_cast<int32_t *>(ws + lay.sorted);
    float *ys = reinterpret_cast<float *>(ws + lay.ys);

    // up to kFusedLoopMax tokens: the fused one-token kernels (gate/up with the
    // shared rows, down with the router-order sum and the epilogue) once per
    // token, in token order, each writing its own output row; the workspace
    // regions they use are reused, stream order keeping the passes apart.
    // The ids and weights are only read (no routing here).
    if (T <= kFusedLoopMax && decode_fused_ok(L)) {
        for (int t = 0; t < T; ++t) {
            OutEpi et = epi;
            if (et.ob) et.ob += (size_t)t * L.H;
            const hipError_t e = launch_decode_fused(L, x + (size_t)t * L.H, const_cast<int32_t *>(idx + (size_t)t * L.K),
                                                     const_cast<float *>(w + (size_t)t * L.K), nullptr, false,
                                                     out + (size_t)t * L.H, ws, lay, s, prof, et, false);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // shapes the fused kernels do not take: the single-token kernels once per
    // token, each writing its token's staging rows of ys, then one combine
    if (T == 1 && decode_path_ok(L))
        return launch_forward_t1(L, x, x, nullptr, idx, w, out, reinterpret_cast<float *>(ws + lay.act),
                                 reinterpret_cast<float *>(ws + lay.ash), ws + lay.ys, nullptr, s, prof, epi);
    if (T <= kT1LoopMax && decode_path_ok(L)) {
        for (int t = 0; t < T; ++t) {
            const uint16_t *xt = x + (size_t)t * L.H;
            const hipError_t e = launch_forward_t1(L, xt, xt, nullptr, idx + (size_t)t * L.K, nullptr, nullptr,
                                                   reinterpret_cast<float *>(ws + lay.act),
                                                   reinterpret_cast<float *>(ws + lay.ash),
                                                   reinterpret_cast<char *>(ys + (size_t)t * (L.K + 1) * L.H),
                                                   nullptr, s, prof, OutEpi());
            if (e != hipSuccess) return e;
        }
        StageMark m(prof, K3MOE_STAGE_COMBINE, s);
        launch_combine(L, ys, w, idx, T, L.H, L.Is > 0, out, s, epi);
        return hipGetLastError();
    }
    launch_perm(L, idx, T, ws, lay, s, prof);
    // activations: routed bf16 hi and lo [T*k][I] in the fp8-term region
    // (4 bytes per element either way); shared bf16 hi and lo [T][Is] in the
    // fp32 shared-activation region
    uint16_t *act_hi = reinterpret_cast<uint16_t *>(ws + lay.act);
    uint16_t *act_lo = act_hi + (size_t)T * L.K * L.I;
    uint16_t *ash_hi = reinterpret_cast<uint16_t *>(ws + lay.ash);
    uint16_t *ash_lo = ash_hi + (size_t)T * L.Is;
    hipError_t e = launch_grouped(L, x, x, nullptr, T, active_n, active_e, active_off, sorted, act_hi, act_lo,
                                  ash_hi, ash_lo, reinterpret_cast<float *>(ws + lay.sh_part),
                                  reinterpret_cast<int2 *>(ws + lay.tiles_gu),
                                  reinterpret_cast<int2 *>(ws + lay.tiles_dn),
                                  reinterpret_cast<int32_t *>(ws + lay.light),
                                  reinterpret_cast<int32_t *>(ws + lay.tile_n), ys, nullptr, s, prof,
                                  term_bufs(ws, lay));
    if (e != hipSuccess) return e;
    {
        StageMark m(prof, K3MOE_STAGE_COMBINE, s);
        launch_combine(L, ys, w, idx, T, L.H, L.Is > 0, out, s, epi);
    }
    return hipGetLastError();
}

}  // namespace k3moe
