// gfx950 grouped GEMMs of the expert layer for batches of tokens (T > 1).
//
// What is computed follows the "kimi-k3-in-c" README, §9 "Picking 16 experts
// of 896" (k3_moe steps 3 and 6, k3_situ_glu) on the MXFP4 format of §4
// "Reduction one: the experts already ship at half a byte".
//
// Design. Once several tokens share an expert the projections are GEMMs:
// for an active expert e with n_e assignments, G = W1_e X_e^T, U = W3_e X_e^T
// (I x n_e), A_e = act(G, U), Y_e = W2_e A_e (H x n_e). They run on the bf16
// MFMA v_mfma_f32_16x16x32_bf16 (products exact, fp32 accumulation):
//  * the fp4 weights are expanded to bf16 in registers with
//    v_cvt_scalef32_pk_bf16_fp4, which applies the block's E8M0 scale
//    exactly (2^(s-127), byte 0 included; byte 255 makes the group zero),
//    so a weight is the exact value the MXFP4 format defines;
//  * the token activations x are bf16 already: one B operand, exact;
//  * the expert activation a (fp32) is fed as two bf16 terms hi + lo
//    (hi = bf16(a), lo = bf16(a - hi); |a - hi - lo| <= 2^-17 |a|), each a
//    separate MFMA into the same accumulator.
// A block owns 256 rows of one expert and a tile of its tokens; weights and
// token rows pass through double-buffered LDS (one barrier per K chunk), the
// next chunk's global loads in flight while the current one is multiplied.
// The shared expert (bf16 weights) runs on the same kernels with the weight
// rows loaded as bf16.
//
// The expert outputs go to the staging rows ys[t][j][.] (and ys[t][k][.] for
// the shared expert); the combine sums them in router order.
#include "k3moe_internal.h"

namespace k3moe {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int kGRows = 256;     // weight rows per block
constexpr int kGWaves = 8;      // 4 row groups (64 rows) x 2 token groups
constexpr int kGuTok = 128;     // tokens per gate/up block (64 per wave)
constexpr int kDnTok = 64;      // tokens per down block (32 per wave)
constexpr int kARowB = 80;      // LDS bytes per weight row per chunk (64 + 16 pad)
constexpr int kBPad = 16;       // LDS padding per token row

__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// E8M0 byte -> fp32 scale for the converter: 2^(s-127); byte 0 is the
// subnormal 2^-127; byte 255 drops its group (scale 0).
__device__ __forceinline__ float e8m0_scale(uint32_t s)
{
    return s == 255u ? 0.0f : __uint_as_float(s == 0u ? 0x00400000u : s << 23);
}

// 8 fp4 weights (one 32-bit word, low nibble first) -> 8 bf16, scaled.
__device__ __forceinline__ bf8 dequant8(uint32_t w, float scale)
{
    const bf2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf8 as_bf8(u4 v)
{
    bf8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ v4f mfma_bf16(const bf8 &a, const bf8 &b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Gated activation (README §9, k3_situ_glu): SiTU-GLU or SwiGLU, fp32.
__device__ __forceinline__ float act_fn(float g, float u, int kind, float b1, float b2)
{
    const float sg = 1.0f / (1.0f + expf(-g));
    if (kind == K3MOE_ACT_SITU) return (b1 * tanhf(g / b1) * sg) * (b2 * tanhf(u / b2));
    return g * sg * u;
}

// ---------------------------------------------------------------------------
// Work lists. Active expert q (ascending id) with n_q assignments goes to the
// gate/up weight-streaming kernel when n_q <= smax_gu (light_gu[] lists such
// q in order), else gets ceil(n_q / bn_gu) GEMM tiles (q, token block); the
// same for the down projection with smax_dn, bn_dn.
// counts: [0] gate/up tiles, [1] down tiles, [2] gate/up light, [3] down light.
__global__ __launch_bounds__(1024) void k_tiles(const int32_t *__restrict__ active_n,
                                                const int32_t *__restrict__ active_off, int bn_gu,
                                                int bn_dn, int smax_gu, int smax_dn,
                                                int2 *__restrict__ tiles_gu, int2 *__restrict__ tiles_dn,
                                                int32_t *__restrict__ light_gu, int32_t *__restrict__ light_dn,
                                                int32_t *counts)
{
    __shared__ int wsum[4][16];
    const int n = *active_n;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (n + 1023) / 1024;
    const int q0 = tid * per;
    int cnt[4] = {0, 0, 0, 0};
    for (int i = 0; i < per; ++i) {
        const int q = q0 + i;
        if (q < n) {
            const int m = active_off[q + 1] - active_off[q];
            if (m <= smax_gu) cnt[2] += 1;
            else cnt[0] += (m + bn_gu - 1) / bn_gu;
            if (m <= smax_dn) cnt[3] += 1;
            else cnt[1] += (m + bn_dn - 1) / bn_dn;
        }
    }
    int inc[4] = {cnt[0], cnt[1], cnt[2], cnt[3]};  // inclusive scans across the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int a = __shfl_up(inc[k], o);
            if (lane >= o) inc[k] += a;
        }
    }
    if (lane == 63)
        for (int k = 0; k < 4; ++k) wsum[k][wv] = inc[k];
    __syncthreads();
    if (tid == 0) {
        for (int k = 0; k < 4; ++k) {
            int r = 0;
            for (int w = 0; w < 16; ++w) {
                const int a = wsum[k][w];
                wsum[k][w] = r;
                r += a;
            }
            counts[k] = r;
        }
    }
    __syncthreads();
    int bg = wsum[0][wv] + inc[0] - cnt[0], bd = wsum[1][wv] + inc[1] - cnt[1];
    int lg = wsum[2][wv] + inc[2] - cnt[2], ld = wsum[3][wv] + inc[3] - cnt[3];
    for (int i = 0; i < per; ++i) {
        const int q = q0 + i;
        if (q < n) {
            const int m = active_off[q + 1] - active_off[q];
            if (m <= smax_gu) light_gu[lg++] = q;
            else
                for (int tb = 0; tb * bn_gu < m; ++tb) tiles_gu[bg++] = int2{q, tb};
            if (m <= smax_dn) light_dn[ld++] = q;
            else
                for (int tb = 0; tb * bn_dn < m; ++tb) tiles_dn[bd++] = int2{q, tb};
        }
    }
}

// ---------------------------------------------------------------------------
// Gate/up GEMM. FP4: routed experts, tile from the list; else the shared
// expert (bf16 weights), token block = blockIdx / RB in token order.
// Chunk = 64 bytes of weight row: 128 K (fp4) or 32 K (bf16).
struct GuGemmParams {
    int H, I, K, T, act;
    float b1, b2;
    const uint8_t *gp, *gs, *up, *us;     // routed fp4 gate/up
    int64_t g_sp, g_ss, u_sp, u_ss;
    const uint16_t *wg, *wu;              // shared bf16 gate/up [I][H]
    const uint16_t *x;                    // bf16 [T][H]
    const int32_t *active_e, *active_off, *sorted;
    const int2 *tiles;
    const int32_t *tile_n;
    uint16_t *act_hi, *act_lo;            // bf16 [rows of assignments / tokens][I]
};

template <bool FP4>
__host__ __device__ constexpr int gu_gemm_lds_bytes()
{
    return 2 * (2 * kGRows * kARowB + (FP4 ? 2 * kGRows * 4 : 0) +
                kGuTok * ((FP4 ? 256 : 64) + kBPad)) +
           kGuTok * 4;
}

template <bool FP4>
__global__ __launch_bounds__(64 * kGWaves) void k_gu_gemm(GuGemmParams p)
{
    constexpr int KC = FP4 ? 128 : 32;          // K elements per chunk
    constexpr int SPC = KC / 32;                // MFMA steps per chunk
    constexpr int BROW = KC * 2 + kBPad;        // LDS bytes per token row
    constexpr int ABUF = 2 * kGRows * kARowB;   // one A buffer (gate + up)
    constexpr int SBUF = FP4 ? 2 * kGRows * 4 : 0;
    constexpr int BBUF = kGuTok * BROW;
    const int H = p.H, I = p.I, RB = (I + kGRows - 1) / kGRows;
    const int tile = blockIdx.x / RB, rb = blockIdx.x - tile * RB;
    const int nrows = min(kGRows, I - rb * kGRows);  // a multiple of 64 (I % 128 == 0)
    int e = 0, p0, n;
    if constexpr (FP4) {
        if (tile >= *p.tile_n) return;
        const int2 tl = p.tiles[tile];
        e = p.active_e[tl.x];
        p0 = p.active_off[tl.x] + tl.y * kGuTok;
        n = min(kGuTok, p.active_off[tl.x + 1] - p0);
    } else {
        p0 = tile * kGuTok;
        n = min(kGuTok, p.T - p0);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;  // row group, token group
    const int g = lane >> 4, l16 = lane & 15;

    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *A_l = lds;                        // [2 bufs][2 mats][256 rows][80 B]
    uint8_t *S_l = A_l + 2 * ABUF;             // [2 bufs][2 mats][256 rows][4 B] (fp4)
    uint8_t *B_l = S_l + 2 * SBUF;             // [2 bufs][128 tokens][BROW]
    int *tok_l = reinterpret_cast<int *>(B_l + 2 * BBUF);  // [128] token of each column

    for (int c = tid; c < kGuTok; c += 64 * kGWaves) {
        const int cc = min(c, n - 1);
        tok_l[c] = FP4 ? p.sorted[p0 + cc] / p.K : p0 + cc;
    }
    __syncthreads();

    // weight rows of this block
    const size_t rowb = FP4 ? (size_t)H / 2 : (size_t)H * 2;  // bytes per weight row
    const uint8_t *wbase[2];
    const uint8_t *sbase[2] = {nullptr, nullptr};
    if constexpr (FP4) {
        wbase[0] = p.gp + e * p.g_sp + (size_t)rb * kGRows * rowb;
        wbase[1] = p.up + e * p.u_sp + (size_t)rb * kGRows * rowb;
        sbase[0] = p.gs + e * p.g_ss + (size_t)rb * kGRows * (H / 32);
        sbase[1] = p.us + e * p.u_ss + (size_t)rb * kGRows * (H / 32);
    } else {
        wbase[0] = reinterpret_cast<const uint8_t *>(p.wg) + (size_t)rb * kGRows * rowb;
        wbase[1] = reinterpret_cast<const uint8_t *>(p.wu) + (size_t)rb * kGRows * rowb;
    }
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(p.x);

    // staging of chunk c: A = 2 mats x 256 rows x 4 u4; S = 512 dwords; B = 128 tokens x (KC*2/16) u4
    constexpr int BSEG = KC * 2 / 16;  // u4 per token row per chunk
    u4 ra[4], rbv[(kGuTok * BSEG + 511) / 512];
    uint32_t rs = 0;
    auto gload = [&](int c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = tid + 512 * q;  // 0..2047
            const int mat = v >> 10, row = min((v >> 2) & 255, nrows - 1), seg = v & 3;
            ra[q] = *reinterpret_cast<const u4 *>(wbase[mat] + (size_t)row * rowb + (size_t)c * 64 + 16 * seg);
        }
        if constexpr (FP4) {
            const int mat = tid >> 8, row = min(tid & 255, nrows - 1);
            rs = *reinterpret_cast<const uint32_t *>(sbase[mat] + (size_t)row * (H / 32) + 4 * c);
        }
#pragma unroll
        for (int q = 0; q < (kGuTok * BSEG + 511) / 512; ++q) {
            const int v = tid + 512 * q;
            const int col = v / BSEG, seg = v - col * BSEG;
            rbv[q] = *reinterpret_cast<const u4 *>(xb + ((size_t)tok_l[col] * H + (size_t)c * KC) * 2 + 16 * seg);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = tid + 512 * q;
            const int mat = v >> 10, row = (v >> 2) & 255, seg = v & 3;
            *reinterpret_cast<u4 *>(A_l + buf * ABUF + (mat * kGRows + row) * kARowB + 16 * seg) = ra[q];
        }
        if constexpr (FP4) *reinterpret_cast<uint32_t *>(S_l + buf * SBUF + 4 * tid) = rs;
#pragma unroll
        for (int q = 0; q < (kGuTok * BSEG + 511) / 512; ++q) {
            const int v = tid + 512 * q;
            const int col = v / BSEG, seg = v - col * BSEG;
            *reinterpret_cast<u4 *>(B_l + buf * BBUF + col * BROW + 16 * seg) = rbv[q];
        }
    };

    // this wave: rows wm*64 + 16 rf + l16; token columns wn*64 + 16 tf + l16
    // token fragments with data (none if the wave's 64 rows are past the end)
    const int ntf = wm * 64 < nrows ? min(4, max(0, (n - wn * 64 + 15) / 16)) : 0;
    v4f acc[2][4][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rf = 0; rf < 4; ++rf)
#pragma unroll
            for (int tf = 0; tf < 4; ++tf) acc[m][rf][tf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int NCH = H / KC;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int c = 0; c < NCH; ++c) {
        const int buf = c & 1;
        if (c + 1 < NCH) gload(c + 1);
        if (ntf > 0) {
            const uint8_t *Ab = A_l + buf * ABUF;
            const uint8_t *Bb = B_l + buf * BBUF;
            uint32_t s4[2][4];  // E8M0 bytes of the chunk's 4 steps, per row fragment
            if constexpr (FP4) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int rf = 0; rf < 4; ++rf) {
                        const int row = wm * 64 + 16 * rf + l16;
                        s4[m][rf] = *reinterpret_cast<const uint32_t *>(S_l + buf * SBUF + 4 * (m * kGRows + row));
                    }
            }
#pragma unroll
            for (int st = 0; st < SPC; ++st) {
                bf8 b[4];
#pragma unroll
                for (int tf = 0; tf < 4; ++tf) {
                    const int col = wn * 64 + 16 * tf + l16;
                    b[tf] = as_bf8(*reinterpret_cast<const u4 *>(Bb + col * BROW + 64 * st + 16 * g));
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    bf8 a[4];
#pragma unroll
                    for (int rf = 0; rf < 4; ++rf) {
                        const int row = wm * 64 + 16 * rf + l16;
                        const uint8_t *ar = Ab + (m * kGRows + row) * kARowB;
                        if constexpr (FP4)
                            a[rf] = dequant8(*reinterpret_cast<const uint32_t *>(ar + 16 * st + 4 * g),
                                             e8m0_scale((s4[m][rf] >> (8 * st)) & 0xffu));
                        else
                            a[rf] = as_bf8(*reinterpret_cast<const u4 *>(ar + 16 * g));
                    }
#pragma unroll
                    for (int tf = 0; tf < 4; ++tf)
                        if (tf < ntf)
#pragma unroll
                            for (int rf = 0; rf < 4; ++rf) acc[m][rf][tf] = mfma_bf16(a[rf], b[tf], acc[m][rf][tf]);
                }
            }
        }
        if (c + 1 < NCH) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: act(g, u) -> bf16 hi + lo, rows of this token column
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
        const int col = wn * 64 + 16 * tf + l16;
        if (tf < ntf && col < n) {
            const size_t orow = (size_t)(p0 + col) * I + (size_t)rb * kGRows;
#pragma unroll
            for (int rf = 0; rf < 4; ++rf) {
                const int row = wm * 64 + 16 * rf + 4 * g;
                uint32_t hi2[2], lo2[2];
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float a0 = act_fn(acc[0][rf][tf][r], acc[1][rf][tf][r], p.act, p.b1, p.b2);
                    const float a1 = act_fn(acc[0][rf][tf][r + 1], acc[1][rf][tf][r + 1], p.act, p.b1, p.b2);
                    const uint16_t h0 = bf16_rne(a0), h1 = bf16_rne(a1);
                    const uint16_t q0 = bf16_rne(a0 - bf16f(h0)), q1 = bf16_rne(a1 - bf16f(h1));
                    hi2[r / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                    lo2[r / 2] = (uint32_t)q0 | ((uint32_t)q1 << 16);
                }
                *reinterpret_cast<uint2 *>(p.act_hi + orow + row) = uint2{hi2[0], hi2[1]};
                *reinterpret_cast<uint2 *>(p.act_lo + orow + row) = uint2{lo2[0], lo2[1]};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Down GEMM: rows of H, tokens of one expert (or the shared expert), the
// activation fed as bf16 hi and lo (two MFMAs into one accumulator).
struct DnGemmParams {
    int H, I, K, T;
    const uint8_t *dp, *ds;               // routed fp4 down [E][H][I/2], scales
    int64_t d_sp, d_ss;
    const uint16_t *wd;                   // shared bf16 down [H][I]
    const uint16_t *act_hi, *act_lo;      // [rows][I]
    const int32_t *active_e, *active_off, *sorted;
    const int2 *tiles;
    const int32_t *tile_n;
    float *ys;                            // [T][K+1][H]
};

template <bool FP4>
__host__ __device__ constexpr int dn_gemm_lds_bytes()
{
    return 2 * (kGRows * kARowB + (FP4 ? kGRows * 4 : 0) + 2 * kDnTok * ((FP4 ? 256 : 64) + kBPad)) +
           kDnTok * 4 * 2;
}

template <bool FP4>
__global__ __launch_bounds__(64 * kGWaves) void k_dn_gemm(DnGemmParams p)
{
    constexpr int KC = FP4 ? 128 : 32;
    constexpr int SPC = KC / 32;
    constexpr int BROW = KC * 2 + kBPad;
    constexpr int ABUF = kGRows * kARowB;
    constexpr int SBUF = FP4 ? kGRows * 4 : 0;
    constexpr int BBUF = 2 * kDnTok * BROW;   // hi rows then lo rows
    const int H = p.H, I = p.I, RB = (H + kGRows - 1) / kGRows;
    const int tile = blockIdx.x / RB, rb = blockIdx.x - tile * RB;
    const int nrows = min(kGRows, H - rb * kGRows);  // a multiple of 64 (H % 128 == 0)
    int e = 0, p0, n;
    if constexpr (FP4) {
        if (tile >= *p.tile_n) return;
        const int2 tl = p.tiles[tile];
        e = p.active_e[tl.x];
        p0 = p.active_off[tl.x] + tl.y * kDnTok;
        n = min(kDnTok, p.active_off[tl.x + 1] - p0);
    } else {
        p0 = tile * kDnTok;
        n = min(kDnTok, p.T - p0);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int g = lane >> 4, l16 = lane & 15;

    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *A_l = lds;
    uint8_t *S_l = A_l + 2 * ABUF;
    uint8_t *B_l = S_l + 2 * SBUF;
    int *orow_l = reinterpret_cast<int *>(B_l + 2 * BBUF);  // [64] output row (t*(K+1)+j) of each column
    int *arow_l = orow_l + kDnTok;                          // [64] activation row of each column

    for (int c = tid; c < kDnTok; c += 64 * kGWaves) {
        const int cc = min(c, n - 1);
        if constexpr (FP4) {
            const int a = p.sorted[p0 + cc];
            orow_l[c] = (a / p.K) * (p.K + 1) + (a % p.K);
        } else {
            orow_l[c] = (p0 + cc) * (p.K + 1) + p.K;
        }
        arow_l[c] = p0 + cc;
    }
    __syncthreads();

    const size_t rowb = FP4 ? (size_t)I / 2 : (size_t)I * 2;
    const uint8_t *wbase, *sbase = nullptr;
    if constexpr (FP4) {
        wbase = p.dp + e * p.d_sp + (size_t)rb * kGRows * rowb;
        sbase = p.ds + e * p.d_ss + (size_t)rb * kGRows * (I / 32);
    } else {
        wbase = reinterpret_cast<const uint8_t *>(p.wd) + (size_t)rb * kGRows * rowb;
    }
    const uint8_t *hib = reinterpret_cast<const uint8_t *>(p.act_hi);
    const uint8_t *lob = reinterpret_cast<const uint8_t *>(p.act_lo);

    constexpr int BSEG = KC * 2 / 16;
    constexpr int NB = (2 * kDnTok * BSEG + 511) / 512;
    u4 ra[2], rbv[NB];
    uint32_t rs = 0;
    auto gload = [&](int c) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int v = tid + 512 * q;  // 0..1023
            const int row = min(v >> 2, nrows - 1), seg = v & 3;
            ra[q] = *reinterpret_cast<const u4 *>(wbase + (size_t)row * rowb + (size_t)c * 64 + 16 * seg);
        }
        if constexpr (FP4) {
            const int row = min(tid & 255, nrows - 1);
            rs = *reinterpret_cast<const uint32_t *>(sbase + (size_t)row * (I / 32) + 4 * c);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + 512 * q;
            const int half = v / (kDnTok * BSEG), vv = v - half * (kDnTok * BSEG);
            const int col = vv / BSEG, seg = vv - col * BSEG;
            const uint8_t *src = half ? lob : hib;
            rbv[q] = *reinterpret_cast<const u4 *>(src + ((size_t)arow_l[col] * I + (size_t)c * KC) * 2 + 16 * seg);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int v = tid + 512 * q;
            const int row = v >> 2, seg = v & 3;
            *reinterpret_cast<u4 *>(A_l + buf * ABUF + row * kARowB + 16 * seg) = ra[q];
        }
        if constexpr (FP4)
            if (tid < kGRows) *reinterpret_cast<uint32_t *>(S_l + buf * SBUF + 4 * tid) = rs;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + 512 * q;
            const int half = v / (kDnTok * BSEG), vv = v - half * (kDnTok * BSEG);
            const int col = vv / BSEG, seg = vv - col * BSEG;
            *reinterpret_cast<u4 *>(B_l + buf * BBUF + (half * kDnTok + col) * BROW + 16 * seg) = rbv[q];
        }
    };

    const int ntf = wm * 64 < nrows ? min(2, max(0, (n - wn * 32 + 15) / 16)) : 0;
    v4f acc[4][2];
#pragma unroll
    for (int rf = 0; rf < 4; ++rf)
#pragma unroll
        for (int tf = 0; tf < 2; ++tf) acc[rf][tf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int NCH = I / KC;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int c = 0; c < NCH; ++c) {
        const int buf = c & 1;
        if (c + 1 < NCH) gload(c + 1);
        if (ntf > 0) {
            const uint8_t *Ab = A_l + buf * ABUF;
            const uint8_t *Bb = B_l + buf * BBUF;
            uint32_t s4[4];
            if constexpr (FP4) {
#pragma unroll
                for (int rf = 0; rf < 4; ++rf) {
                    const int row = wm * 64 + 16 * rf + l16;
                    s4[rf] = *reinterpret_cast<const uint32_t *>(S_l + buf * SBUF + 4 * row);
                }
            }
#pragma unroll
            for (int st = 0; st < SPC; ++st) {
                bf8 a[4];
#pragma unroll
                for (int rf = 0; rf < 4; ++rf) {
                    const int row = wm * 64 + 16 * rf + l16;
                    const uint8_t *ar = Ab + row * kARowB;
                    if constexpr (FP4)
                        a[rf] = dequant8(*reinterpret_cast<const uint32_t *>(ar + 16 * st + 4 * g),
                                         e8m0_scale((s4[rf] >> (8 * st)) & 0xffu));
                    else
                        a[rf] = as_bf8(*reinterpret_cast<const u4 *>(ar + 16 * g));
                }
#pragma unroll
                for (int tf = 0; tf < 2; ++tf) {
                    if (tf < ntf) {
                        const int col = wn * 32 + 16 * tf + l16;
                        const bf8 bh = as_bf8(*reinterpret_cast<const u4 *>(Bb + col * BROW + 64 * st + 16 * g));
                        const bf8 bl = as_bf8(*reinterpret_cast<const u4 *>(Bb + (kDnTok + col) * BROW + 64 * st + 16 * g));
#pragma unroll
                        for (int rf = 0; rf < 4; ++rf) {
                            acc[rf][tf] = mfma_bf16(a[rf], bh, acc[rf][tf]);
                            acc[rf][tf] = mfma_bf16(a[rf], bl, acc[rf][tf]);
                        }
                    }
                }
            }
        }
        if (c + 1 < NCH) lstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int tf = 0; tf < 2; ++tf) {
        const int col = wn * 32 + 16 * tf + l16;
        if (tf < ntf && col < n) {
            float *yr = p.ys + (size_t)orow_l[col] * H + (size_t)rb * kGRows;
#pragma unroll
            for (int rf = 0; rf < 4; ++rf) {
                const int row = wm * 64 + 16 * rf + 4 * g;
                *reinterpret_cast<float4 *>(yr + row) =
                    float4{acc[rf][tf][0], acc[rf][tf][1], acc[rf][tf][2], acc[rf][tf][3]};
            }
        }
    }
}

}  // namespace

// Launch-time limits of the grouped kernels (hidden, inter, shared inter are
// validated multiples of 128 at layer creation).
static bool set_lds_limits()
{
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gu_gemm<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gu_gemm_lds_bytes<true>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gu_gemm<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gu_gemm_lds_bytes<false>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_dn_gemm<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, dn_gemm_lds_bytes<true>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_dn_gemm<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, dn_gemm_lds_bytes<false>());
    return true;
}

size_t grouped_tile_cap(int64_t T, int K, int E, int bn)
{
    return (size_t)(T * K / bn + std::min<int64_t>(E, T * K) + 1);
}

size_t grouped_tile_cap_gu(int64_t T, int K, int E) { return grouped_tile_cap(T, K, E, kGuTok); }
size_t grouped_tile_cap_dn(int64_t T, int K, int E) { return grouped_tile_cap(T, K, E, kDnTok); }

hipError_t launch_grouped(const LayerView &L, const uint16_t *x, int T, const int32_t *active_n,
                          const int32_t *active_e, const int32_t *active_off, const int32_t *sorted,
                          uint16_t *act_hi, uint16_t *act_lo, uint16_t *ash_hi, uint16_t *ash_lo,
                          int2 *tiles_gu, int2 *tiles_dn, int32_t *light, int32_t *counts, float *ys,
                          hipStream_t s, Profiler *prof)
{
    static const bool lds_set = set_lds_limits();  // once per process (thread-safe static)
    (void)lds_set;
    const size_t cap_gu = grouped_tile_cap(T, L.K, L.E, kGuTok), cap_dn = grouped_tile_cap(T, L.K, L.E, kDnTok);
    const int rb_i = (L.I + kGRows - 1) / kGRows, rb_h = (L.H + kGRows - 1) / kGRows;
    const int rb_s = (L.Is + kGRows - 1) / kGRows;
    const bool stream = stream_path_ok(L), stream_dn = stream_down_ok(L);
    const bool sh_stream = stream_shared_ok(L, T);
    int32_t *light_gu = light, *light_dn = light + L.E;
    k_tiles<<<1, 1024, 0, s>>>(active_n, active_off, kGuTok, kDnTok, stream ? stream_max_tokens() : 0,
                               stream_dn ? stream_max_tokens() : 0, tiles_gu, tiles_dn, light_gu, light_dn, counts);

    GuGemmParams gp{};
    gp.H = L.H;
    gp.I = L.I;
    gp.K = L.K;
    gp.T = T;
    gp.act = L.act;
    gp.b1 = L.b1;
    gp.b2 = L.b2;
    gp.gp = L.gp;
    gp.gs = L.gs;
    gp.up = L.up;
    gp.us = L.us;
    gp.g_sp = L.g_sp;
    gp.g_ss = L.g_ss;
    gp.u_sp = L.u_sp;
    gp.u_ss = L.u_ss;
    gp.x = x;
    gp.active_e = active_e;
    gp.active_off = active_off;
    gp.sorted = sorted;
    gp.tiles = tiles_gu;
    gp.tile_n = counts;
    gp.act_hi = act_hi;
    gp.act_lo = act_lo;
    {
        StageMark m(prof, K3MOE_STAGE_GATEUP, s);
        if (stream) {
            const hipError_t e = launch_stream_gu(L, x, T, active_e, active_off, sorted, light_gu, counts + 2,
                                                  sh_stream, act_hi, act_lo, ash_hi, ash_lo, s);
            if (e != hipSuccess) return e;
        }
        const unsigned nblk = (unsigned)(cap_gu * rb_i);
        k_gu_gemm<true><<<nblk, 64 * kGWaves, gu_gemm_lds_bytes<true>(), s>>>(gp);
    }
    if (L.Is > 0 && !sh_stream) {
        StageMark m(prof, K3MOE_STAGE_SHARED_GATEUP, s);
        GuGemmParams sp = gp;
        sp.I = L.Is;
        sp.wg = L.sh_gate;
        sp.wu = L.sh_up;
        sp.act_hi = ash_hi;
        sp.act_lo = ash_lo;
        const unsigned nblk = (unsigned)(((T + kGuTok - 1) / kGuTok) * rb_s);
        k_gu_gemm<false><<<nblk, 64 * kGWaves, gu_gemm_lds_bytes<false>(), s>>>(sp);
    }

    DnGemmParams dp{};
    dp.H = L.H;
    dp.I = L.I;
    dp.K = L.K;
    dp.T = T;
    dp.dp = L.dp;
    dp.ds = L.ds;
    dp.d_sp = L.d_sp;
    dp.d_ss = L.d_ss;
    dp.act_hi = act_hi;
    dp.act_lo = act_lo;
    dp.active_e = active_e;
    dp.active_off = active_off;
    dp.sorted = sorted;
    dp.tiles = tiles_dn;
    dp.tile_n = counts + 1;
    dp.ys = ys;
    {
        StageMark m(prof, K3MOE_STAGE_DOWN, s);
        if (stream_dn) {
            const hipError_t e = launch_stream_dn(L, T, active_e, active_off, sorted, light_dn, counts + 3,
                                                  sh_stream, act_hi, act_lo, ash_hi, ash_lo, ys, s);
            if (e != hipSuccess) return e;
        }
        const unsigned nblk = (unsigned)(cap_dn * rb_h);
        k_dn_gemm<true><<<nblk, 64 * kGWaves, dn_gemm_lds_bytes<true>(), s>>>(dp);
        if (L.Is > 0 && !sh_stream) {
            DnGemmParams sp = dp;
            sp.I = L.Is;
            sp.wd = L.sh_down;
            sp.act_hi = ash_hi;
            sp.act_lo = ash_lo;
            const unsigned nb2 = (unsigned)(((T + kDnTok - 1) / kDnTok) * rb_h);
            k_dn_gemm<false><<<nb2, 64 * kGWaves, dn_gemm_lds_bytes<false>(), s>>>(sp);
        }
    }
    return hipGetLastError();
}

}  // namespace k3moe
