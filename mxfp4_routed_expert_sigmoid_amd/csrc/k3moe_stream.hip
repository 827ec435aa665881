// gfx950 weight-streaming kernels for experts that hold few tokens (T > 1).
//
// What is computed follows the "kimi-k3-in-c" README, §9 "Picking 16 experts
// of 896" (k3_moe steps 3 and 6, k3_situ_glu) on the MXFP4 format of §4
// "Reduction one: the experts already ship at half a byte".
//
// When an expert holds at most 16 of the batch's assignments its projections
// are bound by streaming its weights, not by the MFMA. Here every wave owns 32
// weight rows (two 16-row MFMA tiles) over the whole K range and all of the
// expert's tokens (one 16-column B tile), so weight bytes go from HBM straight
// into registers, each loaded once, with the next group of K in flight while
// the current one is multiplied. The tokens (bf16 x, or the bf16 hi/lo
// activation planes) pass through LDS, staged one K group ahead by the whole
// block. Products run on v_mfma_f32_16x16x32_bf16 after an exact fp4 -> bf16
// expansion (v_cvt_scalef32_pk_bf16_fp4 applies the E8M0 scale; byte 255
// gives zeros), as in the grouped GEMMs.
//
// K mapping. An MFMA step multiplies 32 K elements; lane group g (lanes
// 16g..16g+15) supplies 8 of them. A lane's 16-byte weight load holds 32
// consecutive fp4 values of its row, i.e. 4 steps' worth for its group: in
// chunk c of a group the lane's group covers K = 128c + 32g + [0, 32) and step
// s takes K = 128c + 32g + 8s + [0, 8). The token side reads the same K from
// LDS, so the sum runs over every K exactly once. For bf16 weights (shared
// expert) a 16-byte load is 8 values, one step: chunk c covers K = 32c + 8g +
// [0, 8).
//
// The same launches also run the shared expert for small batches: its blocks
// come first in the grid (token groups of 16, bf16 weights), so they stream
// alongside the routed blocks.
#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kSWaves = 4;                 // waves per block
constexpr int kSRows = 32;                 // weight rows per wave
constexpr int kSBlkRows = kSWaves * kSRows;
constexpr int kSTok = 16;                  // tokens per stream item (one B tile)
constexpr int kSChunks = 4;                // 16-byte weight loads per row per K group
constexpr int kSPad = 16;                  // LDS padding per token row

// An item's LDS header: per column c < 16 its token (key), the row its
// operand comes from (val), its output row (out), its staged row (cmap); per
// staged row r its source row (src); the staged row count. Columns with the
// same token share one staged row: a token naming an expert twice gets the
// same activations twice, so one staged row per distinct token is exact and
// an item never needs more than min(T, 16) of them.
constexpr int kHdrKey = 0, kHdrVal = 16, kHdrOut = 32, kHdrMap = 48, kHdrSrc = 64, kHdrN = 80;
constexpr int kHdrBytes = 96 * 4;

// Wave 0 (call between barriers): the staged rows of an item whose n
// columns carry non-decreasing keys (the stable sort keeps an expert's
// assignments in token order; a shared item's tokens are consecutive).
__device__ __forceinline__ void item_rows(int *hdr, int n)
{
    if (threadIdx.x < 64) {
        const int c = threadIdx.x;
        const bool in = c < n;
        const bool head = in && (c == 0 || hdr[kHdrKey + c] != hdr[kHdrKey + c - 1]);
        const uint64_t m = __ballot(head);
        if (in) {
            const int r = __popcll(m & ((2ull << c) - 1ull)) - 1;
            hdr[kHdrMap + c] = r;
            if (head) hdr[kHdrSrc + r] = hdr[kHdrVal + c];
        }
        if (c == 0) hdr[kHdrN] = __popcll(m);
    }
}

// K elements per group and token-row bytes per group.
template <bool FP4> constexpr int group_k() { return FP4 ? 128 * kSChunks : 8 * 4 * kSChunks; }
template <bool FP4> constexpr int brow_bytes() { return group_k<FP4>() * 2 + kSPad; }

// ---------------------------------------------------------------------------
// Gate/up.
struct GuStreamParams {
    int H, I, K, T, Is, act;
    float b1, b2;
    const uint8_t *gp, *gs, *up, *us;
    int64_t g_sp, g_ss, u_sp, u_ss;
    const uint16_t *sh_gate, *sh_up;
    const uint16_t *x;        // tokens of the shared expert, bf16 [T][H]
    const uint16_t *xr, *xr_lo;  // tokens of the routed experts, bf16 [T][Kr]; xr_lo: a second plane or null
    int Kr;                   // routed experts' width (H, or the latent)
    const int32_t *active_e, *active_off, *sorted;
    const int32_t *light, *light_n;
    int sh_blocks;            // leading blocks that run the shared expert
    int sh_slices;            // hidden-dimension slices of a shared block (1: whole K)
    float *sh_part;           // sh_slices > 1: fp32 partial sums [slice][T][gate, up][I_s]
    uint16_t *act_hi, *act_lo, *ash_hi, *ash_lo;
    int stg;                  // token rows per plane and buffer in LDS (min(16, T): no item has more)
};

// np: token planes (1, or 2 when the routed tokens come as bf16 hi and lo);
// stg: token rows staged per plane and buffer
constexpr int gu_stream_lds_bytes(int np, int stg) { return 2 * np * stg * brow_bytes<true>() + kHdrBytes; }

// The wave's part of one block: gate and up rows row0 + 16 rf + l16 (rf = 0, 1)
// of an item of n columns whose distinct tokens hdr[kHdrSrc + r] (r <
// hdr[kHdrN] <= p.stg) are staged; column c reads staged row hdr[kHdrMap +
// c] (columns past n read the last column's and are never stored),
// over the K groups [g0, g1). The tokens are NP bf16 planes of width KW
// (xp[0], xp[1]: hi and lo of an fp32 input, multiplied into one
// accumulator). part == null: the activation goes to ohi/olo rows orow0 +
// column; else the fp32 gate and up sums go to part[(orow0 + column) * 2 +
// {0, 1}][row] (a slice's partials).
template <bool FP4, int NP>
__device__ __forceinline__ void gu_stream_block(const GuStreamParams &p, const uint8_t *wg, const uint8_t *wu,
                                                const uint8_t *sg, const uint8_t *su, int rows, int row0,
                                                const int *hdr, int n, uint8_t *B_l, uint16_t *ohi,
                                                uint16_t *olo, int64_t orow0, int ostride, int g0, int g1,
                                                float *part, const uint16_t *x0, const uint16_t *x1, int KW)
{
    constexpr int GK = group_k<FP4>();
    constexpr int BROW = brow_bytes<FP4>();
    constexpr int BU4 = GK * 2 / 16;                           // u4 per token row per group
    constexpr int NB = (kSTok * BU4 + 64 * kSWaves - 1) / (64 * kSWaves);  // staging u4 per thread and plane
    const int H = KW, tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int stg = p.stg, nv = hdr[kHdrN] * BU4;  // staged rows per plane; u4 of the staged rows
    const int brow = hdr[kHdrMap + min(l16, n - 1)];  // the staged row of this lane's B column
    const size_t rowb = FP4 ? (size_t)H / 2 : (size_t)H * 2;
    const uint8_t *wr[2][2];
    const uint8_t *sr[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) {
        const int r = min(row0 + 16 * rf + l16, rows - 1);
        wr[0][rf] = wg + (size_t)r * rowb + 16 * g;
        wr[1][rf] = wu + (size_t)r * rowb + 16 * g;
        if constexpr (FP4) {
            sr[0][rf] = sg + (size_t)r * (H / 32);
            sr[1][rf] = su + (size_t)r * (H / 32);
        }
    }
    const uint8_t *xb[2] = {reinterpret_cast<const uint8_t *>(x0), reinterpret_cast<const uint8_t *>(x1)};

    struct Grp {
        u4 a[2][2][kSChunks];  // [mat][rf][chunk]
        u4 s[2][2];            // FP4: the group's 16 scale bytes per row
    };
    auto gload = [&](int gi, Grp &b) {
        const int gc = min(gi, g1 - 1);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) {
#pragma unroll
                for (int c = 0; c < kSChunks; ++c)
                    b.a[m][rf][c] = *reinterpret_cast<const u4 *>(wr[m][rf] + (size_t)gc * (kSChunks * 64) + 64 * c);
                if constexpr (FP4) b.s[m][rf] = *reinterpret_cast<const u4 *>(sr[m][rf] + 16 * gc);
            }
    };
    u4 xs[NP][NB];
    auto xload = [&](int gi) {
        const int gc = min(gi, g1 - 1);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
            for (int q = 0; q < NB; ++q) {  // unconditional (clamped) loads keep the wait counts exact
                const int v = min(tid + 64 * kSWaves * q, nv - 1);
                const int col = v / BU4, seg = v - col * BU4;
                xs[pl][q] = *reinterpret_cast<const u4 *>(
                    xb[pl] + ((size_t)hdr[kHdrSrc + col] * H + (size_t)gc * GK) * 2 + 16 * seg);
            }
    };
    auto xstore = [&](int buf) {
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int v = tid + 64 * kSWaves * q;
                if (v < nv) {
                    const int col = v / BU4, seg = v - col * BU4;
                    *reinterpret_cast<u4 *>(B_l + ((buf * NP + pl) * stg + col) * BROW + 16 * seg) = xs[pl][q];
                }
            }
    };

    v4f acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) acc[m][rf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const Grp &b, int buf) {
        const uint8_t *Bb = B_l + (buf * NP * stg + brow) * BROW;
#pragma unroll
        for (int c = 0; c < kSChunks; ++c) {
            float sc[2][2];
            if constexpr (FP4) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int rf = 0; rf < 2; ++rf) sc[m][rf] = e8m0_to_f32((b.s[m][rf][c] >> (8 * g)) & 0xffu);
            }
            constexpr int SPC = FP4 ? 4 : 1;  // MFMA steps per 16-byte load
#pragma unroll
            for (int st = 0; st < SPC; ++st) {
                const int kb = FP4 ? (128 * c + 32 * g + 8 * st) : (32 * c + 8 * g);
                bf8 bv[NP];
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    bv[pl] = as_bf8(*reinterpret_cast<const u4 *>(Bb + pl * stg * BROW + 2 * kb));
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int rf = 0; rf < 2; ++rf) {
                        bf8 a;
                        if constexpr (FP4)
                            a = dequant8_bf16(b.a[m][rf][c][st], sc[m][rf]);
                        else
                            a = as_bf8(b.a[m][rf][c]);
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl) acc[m][rf] = mfma_bf16(a, bv[pl], acc[m][rf]);
                    }
            }
        }
    };

    // Token loads go before weight loads: the LDS store of the next token
    // group then waits only for the token loads (memory counters retire in
    // issue order) while the weight loads stay in flight.
    Grp b0, b1;
    xload(g0);
    gload(g0, b0);
    xstore(0);
    __syncthreads();
    for (int gi = g0; gi < g1; gi += 2) {
        xload(gi + 1);
        gload(gi + 1, b1);
        compute(b0, 0);
        xstore(1);
        __syncthreads();
        if (gi + 1 >= g1) break;
        xload(gi + 2);
        gload(gi + 2, b0);
        compute(b1, 1);
        xstore(0);
        __syncthreads();
    }

    if (part) {  // a slice's fp32 partial sums
        if (l16 < n) {
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) {
                const int row = row0 + 16 * rf + 4 * g;
                if (row >= rows) continue;
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    *reinterpret_cast<float4 *>(part + ((size_t)(orow0 + l16) * 2 + m) * rows + row) =
                        float4{acc[m][rf][0], acc[m][rf][1], acc[m][rf][2], acc[m][rf][3]};
            }
        }
        return;
    }
    // epilogue: lane holds rows 4g + i (i = 0..3) of token column l16
    if (l16 < n) {
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) {
            const int row = row0 + 16 * rf + 4 * g;
            if (row >= rows) continue;
            uint32_t hi2[2], lo2[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float a0 = act_fn(acc[0][rf][i], acc[1][rf][i], p.act, p.b1, p.b2);
                const float a1 = act_fn(acc[0][rf][i + 1], acc[1][rf][i + 1], p.act, p.b1, p.b2);
                const uint16_t h0 = bf16_rne(a0), h1 = bf16_rne(a1);
                const uint16_t q0 = bf16_rne(a0 - bf16f(h0)), q1 = bf16_rne(a1 - bf16f(h1));
                hi2[i / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lo2[i / 2] = (uint32_t)q0 | ((uint32_t)q1 << 16);
            }
            const size_t o = (size_t)(orow0 + l16) * ostride + row;
            *reinterpret_cast<uint2 *>(ohi + o) = uint2{hi2[0], hi2[1]};
            *reinterpret_cast<uint2 *>(olo + o) = uint2{lo2[0], lo2[1]};
        }
    }
}

__global__ __launch_bounds__(64 * kSWaves) void k_gu_stream(GuStreamParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    int *hdr = reinterpret_cast<int *>(lds);
    uint8_t *B_l = lds + kHdrBytes;
    const int wave = threadIdx.x >> 6;
    int b = blockIdx.x;
    if (b < p.sh_blocks) {  // shared expert: token group tg, rows [rb*128, rb*128 + 128) of I_s, slice ks
        const int RB = p.Is / kSBlkRows, S = p.sh_slices;
        const int ks = b % S, tb = b / S;
        const int tg = tb / RB, rb = tb - tg * RB;
        const int t0 = tg * kSTok, n = min(kSTok, p.T - t0);
        const int NG = p.H / group_k<false>();
        if (threadIdx.x < kSTok) hdr[kHdrKey + threadIdx.x] = hdr[kHdrVal + threadIdx.x] = t0 + min((int)threadIdx.x, n - 1);
        __syncthreads();
        item_rows(hdr, n);
        __syncthreads();
        gu_stream_block<false, 1>(p, reinterpret_cast<const uint8_t *>(p.sh_gate),
                                  reinterpret_cast<const uint8_t *>(p.sh_up), nullptr, nullptr, p.Is,
                                  rb * kSBlkRows + wave * kSRows, hdr, n, B_l, p.ash_hi, p.ash_lo, t0, p.Is,
                                  NG * ks / S, NG * (ks + 1) / S,
                                  S > 1 ? p.sh_part + (size_t)ks * p.T * 2 * p.Is : nullptr, p.x, nullptr, p.H);
        return;
    }
    b -= p.sh_blocks;
    const int RB = p.I / kSBlkRows;
    const int li = b / RB, rb = b - li * RB;
    if (li >= *p.light_n) return;
    const int q = p.light[li], e = p.active_e[q];
    const int off = p.active_off[q], n = p.active_off[q + 1] - off;
    if (threadIdx.x < kSTok)
        hdr[kHdrKey + threadIdx.x] = hdr[kHdrVal + threadIdx.x] = p.sorted[off + min((int)threadIdx.x, n - 1)] / p.K;
    __syncthreads();
    item_rows(hdr, n);
    __syncthreads();
    if (p.xr_lo)
        gu_stream_block<true, 2>(p, p.gp + e * p.g_sp, p.up + e * p.u_sp, p.gs + e * p.g_ss, p.us + e * p.u_ss,
                                 p.I, rb * kSBlkRows + wave * kSRows, hdr, n, B_l, p.act_hi, p.act_lo, off, p.I,
                                 0, p.Kr / group_k<true>(), nullptr, p.xr, p.xr_lo, p.Kr);
    else
        gu_stream_block<true, 1>(p, p.gp + e * p.g_sp, p.up + e * p.u_sp, p.gs + e * p.g_ss, p.us + e * p.u_ss,
                                 p.I, rb * kSBlkRows + wave * kSRows, hdr, n, B_l, p.act_hi, p.act_lo, off, p.I,
                                 0, p.Kr / group_k<true>(), nullptr, p.xr, nullptr, p.Kr);
}

// Shared expert's slices -> activation: g and u summed over the slices in
// order, act(g, u) as bf16 hi + lo.
__global__ __launch_bounds__(256) void k_sh_act(const float *__restrict__ part, int S, int T, int Is, int act,
                                                float b1, float b2, uint16_t *__restrict__ ash_hi,
                                                uint16_t *__restrict__ ash_lo)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * Is) return;
    const int64_t t = i / Is;
    const int r = (int)(i - t * Is);
    float gs = 0.0f, us = 0.0f;
    for (int k = 0; k < S; ++k) {
        const float *pk = part + ((size_t)k * T + t) * 2 * Is;
        gs += pk[r];
        us += pk[Is + r];
    }
    const float a = act_fn(gs, us, act, b1, b2);
    const uint16_t h = bf16_rne(a);
    ash_hi[i] = h;
    ash_lo[i] = bf16_rne(a - bf16f(h));
}

// ---------------------------------------------------------------------------
// Down: rows of H; the activation fed as bf16 hi and lo (two MFMAs into one
// accumulator); outputs to the staging rows ys[t][j] (shared: ys[t][k]).
// A block of 8 waves stages the item's activation planes for the whole K
// range in LDS once (16 tokens x I x hi/lo), then walks a run of 256-row
// blocks of H; each wave streams its 32 rows per row block, its weight loads
// running one K group ahead across row-block boundaries, with no further
// barriers.
constexpr int kDWaves = 8;
constexpr int kDBlkRows = kDWaves * kSRows;  // 256

struct DnStreamParams {
    int H, I, K, T, Is;
    int Hr;                   // routed experts' output rows (H, or the latent)
    float *ysh;               // shared expert's output fp32 [sh_ks][T][H]; null: ys slot K
    int sh_ks;                // K slices of the shared rows (ysh only): fp32 partial sums
    const uint8_t *dp, *ds;
    int64_t d_sp, d_ss;
    const uint16_t *sh_down;
    const uint16_t *act_hi, *act_lo, *ash_hi, *ash_lo;
    const int32_t *active_e, *active_off, *sorted;
    const int32_t *light, *light_n;
    int sh_items;             // leading items that run the shared expert (token groups)
    int stg;                  // token rows staged per item (min(16, T): no item has more)
    int runs, run_rb;         // blocks per item, 256-row blocks per block
    float *ys;
};

// LDS of a down block: both planes of stg staged token rows of width KD
__host__ __device__ constexpr int dn_stream_lds_bytes(int KD, int stg)
{
    return 2 * stg * (2 * KD + kSPad) + kHdrBytes;
}

// Rows [rb0, rb1) x 256 of an R-row matrix, K columns [k0, k0 + KD) of rows
// KW long (weights and activations), into yout rows orow * R.
template <bool FP4>
__device__ __forceinline__ void dn_stream_run(const DnStreamParams &p, const uint8_t *wd, const uint8_t *sd, int KD,
                                              int rb0, int rb1, const int *hdr, int n,
                                              const uint16_t *ahi, const uint16_t *alo, uint8_t *B_l, int R,
                                              float *yout, int KW, int k0)
{
    constexpr int GK = group_k<FP4>();
    const int BROW = 2 * KD + kSPad;
    const int H = R, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int NG = KD / GK, total = (rb1 - rb0) * NG;
    const size_t rowb = FP4 ? (size_t)KW / 2 : (size_t)KW * 2;
    wd += FP4 ? k0 / 2 : (size_t)k0 * 2;
    if (FP4) sd += k0 / 32;

    // stage both activation planes of the item's staged rows (one per
    // distinct token, at most stg), whole K range
    const int stg = p.stg, nr = hdr[kHdrN];
    {
        const int ru4 = KD * 2 / 16;  // u4 per token row
        for (int v = tid; v < 2 * nr * ru4; v += 64 * kDWaves) {
            const int half = v / (nr * ru4), vv = v - half * (nr * ru4);
            const int col = vv / ru4, seg = vv - col * ru4;
            const uint16_t *src = half ? alo : ahi;
            *reinterpret_cast<u4 *>(B_l + (half * stg + col) * BROW + 16 * seg) =
                *reinterpret_cast<const u4 *>(src + (size_t)hdr[kHdrSrc + col] * KW + k0 + 8 * seg);
        }
    }
    __syncthreads();

    struct Grp {
        u4 a[2][kSChunks];
        u4 s[2];
    };
    auto gload = [&](int it, Grp &b) {
        const int ic = min(it, total - 1);
        const int rb = rb0 + ic / NG, gi = ic - (ic / NG) * NG;
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) {
            const int r = min(rb * kDBlkRows + wave * kSRows + 16 * rf + l16, H - 1);
            const uint8_t *w = wd + (size_t)r * rowb + 16 * g + (size_t)gi * (kSChunks * 64);
#pragma unroll
            for (int c = 0; c < kSChunks; ++c) b.a[rf][c] = *reinterpret_cast<const u4 *>(w + 64 * c);
            if constexpr (FP4) b.s[rf] = *reinterpret_cast<const u4 *>(sd + (size_t)r * (KW / 32) + 16 * gi);
        }
    };

    v4f acc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
    // B column l16 reads its staged row (columns past n repeat the last
    // column's, never stored)
    const int brow = hdr[kHdrMap + min(l16, n - 1)];
    const uint8_t *Bh = B_l + brow * BROW;
    const uint8_t *Bl = B_l + (stg + brow) * BROW;
    auto compute = [&](const Grp &b, int it) {
        const int rb = rb0 + it / NG, gi = it - (it / NG) * NG;
        const int kg = gi * GK;
#pragma unroll
        for (int c = 0; c < kSChunks; ++c) {
            float sc[2];
            if constexpr (FP4) {
#pragma unroll
                for (int rf = 0; rf < 2; ++rf) sc[rf] = e8m0_to_f32((b.s[rf][c] >> (8 * g)) & 0xffu);
            }
            constexpr int SPC = FP4 ? 4 : 1;
#pragma unroll
            for (int st = 0; st < SPC; ++st) {
                const int kb = kg + (FP4 ? (128 * c + 32 * g + 8 * st) : (32 * c + 8 * g));
                const bf8 bh = as_bf8(*reinterpret_cast<const u4 *>(Bh + 2 * kb));
                const bf8 bl = as_bf8(*reinterpret_cast<const u4 *>(Bl + 2 * kb));
#pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    bf8 a;
                    if constexpr (FP4)
                        a = dequant8_bf16(b.a[rf][c][st], sc[rf]);
                    else
                        a = as_bf8(b.a[rf][c]);
                    acc[rf] = mfma_bf16(a, bh, acc[rf]);
                    acc[rf] = mfma_bf16(a, bl, acc[rf]);
                }
            }
        }
        if (gi == NG - 1) {  // row block done: lane holds rows 4g + i of token column l16
            if (l16 < n) {
                float *yr = yout + (size_t)hdr[kHdrOut + l16] * H;
#pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    const int row = rb * kDBlkRows + wave * kSRows + 16 * rf + 4 * g;
                    if (row < H)
                        *reinterpret_cast<float4 *>(yr + row) = float4{acc[rf][0], acc[rf][1], acc[rf][2], acc[rf][3]};
                }
            }
            acc[0] = acc[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    Grp b0, b1;
    gload(0, b0);
    for (int it = 0; it < total; it += 2) {
        gload(it + 1, b1);
        compute(b0, it);
        if (it + 1 >= total) break;
        gload(it + 2, b0);
        compute(b1, it + 1);
    }
}

__global__ __launch_bounds__(64 * kDWaves) void k_dn_stream(DnStreamParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    int *hdr = reinterpret_cast<int *>(lds);
    uint8_t *B_l = lds + kHdrBytes;
    const int item = blockIdx.x / p.runs, run = blockIdx.x - item * p.runs;
    const int R = item < p.sh_items ? p.H : p.Hr;  // output rows of this item
    const int RBT = (R + kDBlkRows - 1) / kDBlkRows;
    const int rb0 = run * p.run_rb, rb1 = min(RBT, rb0 + p.run_rb);
    if (rb0 >= rb1) return;
    if (item < p.sh_items) {  // shared expert: token group tg (p.stg tokens), K slice ks
        const int tg = item / p.sh_ks, ks = item - tg * p.sh_ks;
        const int t0 = tg * p.stg, n = min(p.stg, p.T - t0);
        if (threadIdx.x < kSTok) {
            const int t = t0 + min((int)threadIdx.x, n - 1);
            hdr[kHdrKey + threadIdx.x] = hdr[kHdrVal + threadIdx.x] = t;
            hdr[kHdrOut + threadIdx.x] = p.ysh ? t : t * (p.K + 1) + p.K;
        }
        __syncthreads();
        item_rows(hdr, n);
        __syncthreads();
        const int KS = p.Is / p.sh_ks;
        dn_stream_run<false>(p, reinterpret_cast<const uint8_t *>(p.sh_down), nullptr, KS, rb0, rb1, hdr, n,
                             p.ash_hi, p.ash_lo, B_l, p.H,
                             p.ysh ? p.ysh + (size_t)ks * p.T * p.H : p.ys, p.Is, ks * KS);
        return;
    }
    const int li = item - p.sh_items;
    if (li >= *p.light_n) return;
    const int q = p.light[li], e = p.active_e[q];
    const int off = p.active_off[q], n = p.active_off[q + 1] - off;
    if (threadIdx.x < kSTok) {
        const int c = min((int)threadIdx.x, n - 1);
        const int a = p.sorted[off + c];
        hdr[kHdrKey + threadIdx.x] = a / p.K;  // the token
        hdr[kHdrVal + threadIdx.x] = off + c;  // its activation row
        hdr[kHdrOut + threadIdx.x] = (a / p.K) * (p.K + 1) + a % p.K;
    }
    __syncthreads();
    item_rows(hdr, n);
    __syncthreads();
    dn_stream_run<true>(p, p.dp + e * p.d_sp, p.ds + e * p.d_ss, p.I, rb0, rb1, hdr, n, p.act_hi, p.act_lo, B_l,
                        p.Hr, p.ys, p.I, 0);
}

}  // namespace

bool stream_path_ok(const LayerView &L)
{
    return L.H % group_k<true>() == 0 && L.EK % group_k<true>() == 0 && L.I % group_k<true>() == 0 &&
           L.I % kSBlkRows == 0 && L.H % kSBlkRows == 0 && L.EK % kSBlkRows == 0 && L.Is % kSBlkRows == 0;
}

int stream_max_tokens() { return kSTok; }

// K slices of the shared expert's down rows when its output goes to a
// buffer of its own (a latent layer: fp32 partials summed in order by the
// consumer). For one token group, 8 (or 4, 2) slices so its few row blocks
// (one per 256 rows of H) do not outlast the routed experts' blocks; for
// more tokens, the fewest that keep a slice no wider than the routed K, so
// the shared rows never need more LDS than the routed ones. Each slice a
// multiple of the bf16 K group.
int stream_shared_down_slices(int Lt, int Is, int T, int I)
{
    if (Lt == 0 || Is == 0) return 1;
    if (T <= kSTok) {
        for (int S = 8; S > 1; S /= 2)
            if (Is % (S * group_k<false>()) == 0) return S;
        return 1;
    }
    for (int S = 1; S <= 8; S *= 2)
        if (Is / S <= I && Is % (S * group_k<false>()) == 0) return S;
    return 1;
}

// Token rows the down kernel stages per item: min(16, T), fewer when both
// activation planes of that many rows at the widest K it stages (the routed
// I, or the shared rows' slice) would not fit in LDS. It is also the light
// limit of the down stage (an item never has more distinct tokens than
// assignments) and the shared expert's token-group size. 0: nothing fits.
int stream_down_rows(const LayerView &L, int T)
{
    const int KD = std::max(L.I, L.Is / stream_shared_down_slices(L.Lt, L.Is, T, L.I));
    const int fit = (160 * 1024 - kHdrBytes) / (2 * (2 * KD + kSPad));
    return std::min(std::min(T, kSTok), fit);
}

bool stream_down_ok(const LayerView &L, int T)
{
    return stream_path_ok(L) && stream_down_rows(L, T) >= 1 && (L.Is == 0 || L.Is % group_k<true>() == 0);
}

bool stream_shared_ok(const LayerView &L, int T) { return L.Is > 0 && T <= 8 * kSTok && stream_down_ok(L, T); }

// Slices of the shared expert's hidden dimension for small batches, where
// its few gate/up blocks (one per 128 rows and token group) would otherwise
// outlast the routed experts' blocks.
int stream_shared_slices(int T) { return T <= 2 * kSTok ? 8 : 1; }

hipError_t launch_stream_gu(const LayerView &L, const uint16_t *x, const uint16_t *xr, const uint16_t *xr_lo,
                            int T, const int32_t *active_e, const int32_t *active_off, const int32_t *sorted,
                            const int32_t *light, const int32_t *light_n, bool with_shared, uint16_t *act_hi,
                            uint16_t *act_lo, uint16_t *ash_hi, uint16_t *ash_lo, float *sh_part, hipStream_t s)
{
    static const bool lds_set = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gu_stream),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, gu_stream_lds_bytes(2, kSTok));
        return true;
    }();
    (void)lds_set;
    GuStreamParams p{};
    p.H = L.H;
    p.I = L.I;
    p.K = L.K;
    p.T = T;
    p.Is = L.Is;
    p.act = L.act;
    p.b1 = L.b1;
    p.b2 = L.b2;
    p.gp = L.gp;
    p.gs = L.gs;
    p.up = L.up;
    p.us = L.us;
    p.g_sp = L.g_sp;
    p.g_ss = L.g_ss;
    p.u_sp = L.u_sp;
    p.u_ss = L.u_ss;
    p.sh_gate = L.sh_gate;
    p.sh_up = L.sh_up;
    p.x = x;
    p.xr = xr;
    p.xr_lo = xr_lo;
    p.Kr = L.EK;
    p.active_e = active_e;
    p.active_off = active_off;
    p.sorted = sorted;
    p.light = light;
    p.light_n = light_n;
    p.stg = std::min(T, kSTok);
    p.sh_slices = with_shared ? std::min(stream_shared_slices(T), L.H / group_k<false>()) : 1;  // no empty slice
    p.sh_part = sh_part;
    p.sh_blocks = with_shared ? ((T + kSTok - 1) / kSTok) * (L.Is / kSBlkRows) * p.sh_slices : 0;
    p.act_hi = act_hi;
    p.act_lo = act_lo;
    p.ash_hi = ash_hi;
    p.ash_lo = ash_lo;
    const int64_t cap = std::min<int64_t>(L.E, (int64_t)T * L.K);
    const unsigned nblk = (unsigned)(p.sh_blocks + cap * (L.I / kSBlkRows));
    k_gu_stream<<<nblk, 64 * kSWaves, gu_stream_lds_bytes(xr_lo ? 2 : 1, p.stg), s>>>(p);
    if (with_shared && p.sh_slices > 1) {
        const int64_t n = (int64_t)T * L.Is;
        k_sh_act<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(sh_part, p.sh_slices, T, L.Is, L.act, L.b1, L.b2,
                                                             ash_hi, ash_lo);
    }
    return hipGetLastError();
}

hipError_t launch_stream_dn(const LayerView &L, int T, const int32_t *active_e, const int32_t *active_off,
                            const int32_t *sorted, const int32_t *light, const int32_t *light_n,
                            bool with_shared, const uint16_t *act_hi, const uint16_t *act_lo,
                            const uint16_t *ash_hi, const uint16_t *ash_lo, float *ys, float *ysh, hipStream_t s)
{
    static const bool lds_set = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_dn_stream),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)lds_set;
    DnStreamParams p{};
    p.H = L.H;
    p.Hr = L.EK;
    p.ysh = ysh;
    p.I = L.I;
    p.K = L.K;
    p.T = T;
    p.Is = L.Is;
    p.dp = L.dp;
    p.ds = L.ds;
    p.d_sp = L.d_sp;
    p.d_ss = L.d_ss;
    p.sh_down = L.sh_down;
    p.act_hi = act_hi;
    p.act_lo = act_lo;
    p.ash_hi = ash_hi;
    p.ash_lo = ash_lo;
    p.active_e = active_e;
    p.active_off = active_off;
    p.sorted = sorted;
    p.light = light;
    p.light_n = light_n;
    p.sh_ks = ysh ? stream_shared_down_slices(L.Lt, L.Is, T, L.I) : 1;
    p.stg = stream_down_rows(L, T);
    p.sh_items = with_shared ? (T + p.stg - 1) / p.stg * p.sh_ks : 0;
    // each item's rows in `runs` blocks of run_rb 256-row blocks: about 7 row
    // blocks per run, fewer when there are few items (about 512 blocks)
    const int64_t cap = std::min<int64_t>(L.E, (int64_t)T * L.K);
    const int rbt = (std::max(L.H, L.EK) + kDBlkRows - 1) / kDBlkRows;
    const int64_t items = p.sh_items + cap;
    const int want = (int)std::max<int64_t>((rbt + 6) / 7, (512 + items - 1) / items);
    p.run_rb = (rbt + std::min(want, rbt) - 1) / std::min(want, rbt);
    p.runs = (rbt + p.run_rb - 1) / p.run_rb;
    p.ys = ys;
    const unsigned nblk = (unsigned)((p.sh_items + cap) * p.runs);
    k_dn_stream<<<nblk, 64 * kDWaves, dn_stream_lds_bytes(std::max(L.I, L.Is / p.sh_ks), p.stg), s>>>(p);
    return hipGetLastError();
}

}  // namespace k3moe
