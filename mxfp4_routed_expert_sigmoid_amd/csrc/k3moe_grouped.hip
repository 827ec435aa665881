// gfx950 grouped GEMMs of the expert layer for batches of tokens (T > 1).
//
// What is computed follows the "kimi-k3-in-c" README, §9 "Picking 16 experts
// of 896" (k3_moe steps 3 and 6, k3_situ_glu) on the MXFP4 format of §4
// "Reduction one: the experts already ship at half a byte".
//
// Design. Once several tokens share an expert the projections are GEMMs:
// for an active expert e with n_e assignments, G = W1_e X_e^T, U = W3_e X_e^T
// (I x n_e), A_e = act(G, U), Y_e = W2_e A_e (H x n_e).
//  * Gate/up tiles run on the bf16 MFMA v_mfma_f32_16x16x32_bf16: the fp4
//    weights are expanded to bf16 in registers with
//    v_cvt_scalef32_pk_bf16_fp4, which applies the block's E8M0 scale
//    exactly (2^(s-127), byte 0 included; byte 255 makes the group zero),
//    and the bf16 tokens are the B operand as they are: every product exact,
//    fp32 accumulation.
//  * Down tiles of the routed experts run on the scaled MFMA
//    v_mfma_scale_f32_16x16x128_f8f6f4: the fp4 weight bytes are the A
//    operand as loaded (their E8M0 byte the A scale) and the activation is
//    fed as kTileTerms e4m3 terms with one E8M0 byte per 32-block each, which
//    the gate/up epilogue writes; one MFMA per term into the same
//    accumulator (about 2^-14 of each block's maximum is left out).
//  * Where the streamed down projection reads an expert's activation (or
//    the down tiles cannot use terms), the activation goes as two bf16
//    planes hi + lo (hi = bf16(a), lo = bf16(a - hi); |a - hi - lo| <=
//    2^-17 |a|) on the bf16 MFMA, as does the shared expert (bf16 weights).
// A block owns 256 rows of one expert and a tile of its tokens; each wave
// loads its weight rows from HBM straight into registers (one 16-byte load
// per lane per K chunk, the next chunk in flight while the current one is
// multiplied), and the token side passes through double-buffered LDS, one
// barrier per K chunk.
//
// The expert outputs go to the staging rows ys[t][j][.] (and ys[t][k][.] for
// the shared expert); the combine sums them in router order.
#include <type_traits>

#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kBPad = 16;       // LDS padding per token row
// e4m3 terms of the activation the down tiles take: three leave about 2^-14
// of each 32-block's maximum out (the one-token path keeps kATerms)
constexpr int kTileTerms = 3;

// ---------------------------------------------------------------------------
// Work lists. Active expert q (ascending id) with n_q assignments goes to the
// gate/up weight-streaming kernel when n_q <= smax_gu (light_gu[] lists such
// q in order; with one_gu, those with n_q == 1 or 2 go to light1[] or
// light2[] instead, for the whole-row gate/up kernel), else gets
// ceil(n_q / bn_gu) GEMM tiles (q, token block); the same for the down
// projection with smax_dn, bn_dn.
// counts: [0] gate/up tiles, [1] down tiles, [2] gate/up light, [3] down
// light, [4] gate/up light with one assignment, [5] with two.
constexpr int kTileCounts = 6;
__global__ __launch_bounds__(1024) void k_tiles(const int32_t *__restrict__ active_n,
                                                const int32_t *__restrict__ active_off, int bn_gu,
                                                int bn_dn, int smax_gu, int smax_dn, int one_gu,
                                                int2 *__restrict__ tiles_gu, int2 *__restrict__ tiles_dn,
                                                int32_t *__restrict__ light_gu, int32_t *__restrict__ light_dn,
                                                int32_t *__restrict__ light1, int32_t *__restrict__ light2,
                                                int32_t *counts)
{
    __shared__ int wsum[kTileCounts][16];
    const int n = *active_n;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (n + 1023) / 1024;
    const int q0 = tid * per;
    int cnt[kTileCounts] = {0, 0, 0, 0, 0, 0};
    for (int i = 0; i < per; ++i) {
        const int q = q0 + i;
        if (q < n) {
            const int m = active_off[q + 1] - active_off[q];
            if (m <= smax_gu) cnt[one_gu && m <= 2 ? 3 + m : 2] += 1;
            else cnt[0] += (m + bn_gu - 1) / bn_gu;
            if (m <= smax_dn) cnt[3] += 1;
            else cnt[1] += (m + bn_dn - 1) / bn_dn;
        }
    }
    int inc[kTileCounts] = {cnt[0], cnt[1], cnt[2], cnt[3], cnt[4], cnt[5]};  // inclusive scans across the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int k = 0; k < kTileCounts; ++k) {
            const int a = __shfl_up(inc[k], o);
            if (lane >= o) inc[k] += a;
        }
    }
    if (lane == 63)
        for (int k = 0; k < kTileCounts; ++k) wsum[k][wv] = inc[k];
    __syncthreads();
    if (tid == 0) {
        for (int k = 0; k < kTileCounts; ++k) {
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
    int l1 = wsum[4][wv] + inc[4] - cnt[4], l2 = wsum[5][wv] + inc[5] - cnt[5];
    for (int i = 0; i < per; ++i) {
        const int q = q0 + i;
        if (q < n) {
            const int m = active_off[q + 1] - active_off[q];
            if (m <= smax_gu) {
                if (one_gu && m == 1) light1[l1++] = q;
                else if (one_gu && m == 2) light2[l2++] = q;
                else light_gu[lg++] = q;
            }
            else
                for (int tb = 0; tb * bn_gu < m; ++tb) tiles_gu[bg++] = int2{q, tb};
            if (m <= smax_dn) light_dn[ld++] = q;
            else
                for (int tb = 0; tb * bn_dn < m; ++tb) tiles_dn[bd++] = int2{q, tb};
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM tiles. A block owns 256 weight rows of one expert (or of the
// shared expert) and one tile of its tokens. Each wave owns RF 16-row MFMA
// tiles over the whole K range and all of the tile's tokens (TF 16-column
// fragments), so a weight fragment is loaded from HBM into registers once,
// expanded to bf16 once, and used for every token fragment; the next K chunk's
// weights are in flight while the current one is multiplied. The tokens (x,
// or the activation's hi and lo planes) pass through double-buffered LDS, one
// barrier per chunk.
//
// K mapping (fp4): a lane's 16-byte weight load in chunk c holds K =
// 128c + 32g + [0, 32) of its row (g = lane / 16); MFMA step s uses
// K = 128c + 32g + 8s + [0, 8), and the token side reads the same K from LDS.
// bf16 weights: chunk c, lane group g holds K = 32c + 8g + [0, 8), one step.
// Tile kinds: gate/up on bf16 tokens, down on the activation's hi and lo,
// gate/up on tokens given as hi and lo (a latent layer's fp32 z).
constexpr int kGU = 0, kDN = 1, kGU2 = 2;
template <int KIND> struct GemmShape;
// MINB: blocks per CU the kernel is built for (registers at most 512 / (4 waves
// per SIMD / ... ) per lane)
template <> struct GemmShape<kGU> {   // gate/up: 8 waves x 32 rows, 128 tokens
    static constexpr int WAVES = 8, RF = 2, TF = 8, NMAT = 2, NPL = 1, TOK = 128, MINB = 1;
};
template <> struct GemmShape<kDN> {   // down: 4 waves x 64 rows, 64 tokens (hi, lo)
    static constexpr int WAVES = 4, RF = 4, TF = 4, NMAT = 1, NPL = 2, TOK = 64, MINB = 1;
};
template <> struct GemmShape<kGU2> {  // gate/up, tokens as hi and lo: 8 waves x 32 rows, 64 tokens
    static constexpr int WAVES = 8, RF = 2, TF = 4, NMAT = 2, NPL = 2, TOK = 64, MINB = 1;
};
// The down tile on the scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4: the
// fp4 weights go in as loaded (A operand, the E8M0 byte as the lane's A
// scale) and the activation as kTileTerms e4m3 terms (B operands with their own
// E8M0 bytes), one MFMA per term into the same accumulator.
constexpr int kDN8 = 4;
template <> struct GemmShape<kDN8> {   // down: 4 waves x 64 rows, 64 tokens, the activation as kTileTerms terms
    static constexpr int WAVES = 4, RF = 4, TF = 4, NMAT = 1, NPL = kTileTerms, TOK = 64, MINB = 1;
};
// weight rows per block: waves x 16-row fragments per wave x 16
template <int KIND>
__host__ __device__ constexpr int tile_rows()
{
    return GemmShape<KIND>::WAVES * GemmShape<KIND>::RF * 16;
}
static_assert(GemmShape<kDN8>::TOK == GemmShape<kDN>::TOK, "one tile list serves both down forms");
static_assert(tile_rows<kGU>() == tile_rows<kGU2>() && tile_rows<kDN>() == tile_rows<kDN8>(),
              "one row-block count per projection");
constexpr int kB8Row = 128 + 16;  // LDS bytes per term row per chunk (128 e4m3 codes + padding)

struct GemmParams {
    int rows, KD, K, T, act;   // weight rows (I / I_s or H), reduction length (H or I / I_s), top-k
    float b1, b2;
    // routed fp4 weights per matrix (gate, up | down), per-expert strides
    const uint8_t *wp[2], *ws[2];
    int64_t wsp[2], wss[2];
    // shared expert: bf16 weights [rows][KD] per matrix
    const uint16_t *wb[2];
    // token planes [.][KD] bf16: x (gate/up), or the activation's hi and lo (down)
    const uint16_t *bp[2];
    const int32_t *active_e, *active_off, *sorted;
    const int2 *tiles;
    const int32_t *tile_n;
    // f8 down tiles: the activation as e4m3 terms [row][NPL][KD] and their
    // E8M0 bytes [row][NPL][KD / 32] (row: the sorted assignment)
    const uint8_t *bq, *bsc;
    int sh_blocks;             // leading blocks that run the shared expert, on:
    int sh_rows, sh_KD;        //   its weight rows (I_s or H) and reduction length (H or I_s),
    const uint16_t *sh_bp[2];  //   its token planes [T][sh_KD] (x, or the activation's hi and lo),
    uint16_t *sh_ohi, *sh_olo; //   its activation outputs (gate/up)
    uint16_t *ohi, *olo;       // gate/up: activation hi/lo [row][rows] (null: not written)
    uint8_t *oq, *osc;         // gate/up: activation as kTileTerms e4m3 terms [row][kTileTerms][rows]
                               // and E8M0 bytes [row][kTileTerms][rows / 32] (null: not written)
    float *ys;                 // down: staging [T][K + 1][H]
};

// One buffer of an f8 tile's token side: the term rows, then one scale word
// (4 E8M0 bytes, a chunk's 4 blocks) per term row.
template <int KIND>
__host__ __device__ constexpr int f8_buf_bytes()
{
    using S = GemmShape<KIND>;
    return S::NPL * S::TOK * (kB8Row + 4);
}

template <int KIND>
__host__ __device__ constexpr int gemm_tok_bytes()
{
    using S = GemmShape<KIND>;
    return KIND == kDN8 ? 2 * f8_buf_bytes<KIND>() : 2 * S::NPL * S::TOK * (128 * 2 + kBPad);
}

template <int KIND>
__host__ __device__ constexpr int gemm_lds_bytes()
{
    return gemm_tok_bytes<KIND>() + 2 * GemmShape<KIND>::TOK * 4;
}

// Gate/up epilogue: the activation of this lane's rows row0 + 16 rf + 4 g +
// [0, 4) for token column col, written as bf16 hi and lo planes and/or as
// kTileTerms e4m3 terms. For the terms a wave's 32 rows are one E8M0 block: the
// 4 lanes holding a column (lane groups 0..3) reduce its maximum. Every lane
// runs the split (the shuffles need the whole wave); only columns with a
// token store.
template <int RF>
__device__ __forceinline__ void gu_epilogue(const GemmParams &p, const float (&av)[RF][4], int row0, int g,
                                            int orow, bool store)
{
    const int rows = p.rows;
    if (p.ohi && store) {
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) {
            uint32_t hi2[2], lo2[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const uint16_t h0 = bf16_rne(av[rf][i]), h1 = bf16_rne(av[rf][i + 1]);
                const uint16_t q0 = bf16_rne(av[rf][i] - bf16f(h0)), q1 = bf16_rne(av[rf][i + 1] - bf16f(h1));
                hi2[i / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lo2[i / 2] = (uint32_t)q0 | ((uint32_t)q1 << 16);
            }
            const size_t o = (size_t)orow * rows + row0 + 16 * rf + 4 * g;
            *reinterpret_cast<uint2 *>(p.ohi + o) = uint2{hi2[0], hi2[1]};
            *reinterpret_cast<uint2 *>(p.olo + o) = uint2{lo2[0], lo2[1]};
        }
    }
    if (p.oq) {
        static_assert(RF % 2 == 0, "whole 32-row blocks per wave");
#pragma unroll
        for (int h = 0; h < RF / 2; ++h) {  // the wave's 32-row block h: fragments 2h, 2h + 1
            float r[8];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) r[4 * f + i] = av[2 * h + f][i];
            uint32_t code[kTileTerms][2];
            int sb[kTileTerms];
            split_e4m3_terms<kTileTerms, 8>(
                r, [](float m) {
                    m = fmaxf(m, __shfl_xor(m, 16));
                    return fmaxf(m, __shfl_xor(m, 32));
                },
                code, sb);
            if (store) {
                const int nb = rows >> 5, rb0 = row0 + 32 * h;
#pragma unroll
                for (int t = 0; t < kTileTerms; ++t) {
                    uint8_t *q = p.oq + ((size_t)orow * kTileTerms + t) * rows + rb0 + 4 * g;
#pragma unroll
                    for (int f = 0; f < 2; ++f) *reinterpret_cast<uint32_t *>(q + 16 * f) = code[t][f];
                    if (g == 0) p.osc[((size_t)orow * kTileTerms + t) * nb + (rb0 >> 5)] = (uint8_t)sb[t];
                }
            }
        }
    }
}

// Epilogue of a tile: lane holds rows 4g + i (i = 0..3) of token column
// 16 tf + l16 in each 16-row fragment rf; gate/up writes the activation,
// down its fp32 rows to the staging rows.
template <int KIND, int NMAT, int RF, int TF>
__device__ __forceinline__ void tile_epilogue(const GemmParams &p, const v4f (&acc)[NMAT][RF][TF], int row0, int ntf,
                                              int n, const int *oro_l)
{
    constexpr bool GU = KIND != kDN && KIND != kDN8;
    const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) {
        if (tf >= ntf) break;  // wave-uniform
        const int col = 16 * tf + l16;
        const bool store = col < n;
        if constexpr (GU) {
            float av[RF][4];
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    av[rf][i] = act_fn(acc[0][rf][tf][i], acc[1][rf][tf][i], p.act, p.b1, p.b2);
            gu_epilogue<RF>(p, av, row0, g, oro_l[min(col, n - 1)], store);
        } else if (store) {
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
                *reinterpret_cast<float4 *>(p.ys + (size_t)oro_l[col] * p.rows + row0 + 16 * rf + 4 * g) =
                    float4{acc[0][rf][tf][0], acc[0][rf][tf][1], acc[0][rf][tf][2], acc[0][rf][tf][3]};
        }
    }
}

template <int KIND, bool FP4>
__device__ __forceinline__ void gemm_tile(const GemmParams &p, int e, int rb, int p0, int n, const int *bro_l,
                                          const int *oro_l, uint8_t *B_l)
{
    using S = GemmShape<KIND>;
    constexpr int WAVES = S::WAVES, RF = S::RF, TF = S::TF, NMAT = S::NMAT, NPL = S::NPL, TOK = S::TOK;
    constexpr int NT = 64 * WAVES;
    constexpr int KC = FP4 ? 128 : 32;           // K per chunk
    constexpr int SPC = FP4 ? 4 : 1;             // MFMA steps per chunk
    constexpr int BROW = KC * 2 + kBPad;         // LDS bytes per token row per chunk
    constexpr int BSEG = KC * 2 / 16;            // u4 per token row per chunk
    constexpr int NBU4 = NPL * TOK * BSEG;       // u4 of one chunk's token tile
    constexpr int NB = (NBU4 + NT - 1) / NT;
    constexpr int BBUF = NPL * TOK * BROW;
    const int KD = p.KD, rows = p.rows, NCH = KD / KC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
    constexpr int TR = tile_rows<KIND>();
    const int nrows = min(TR, rows - rb * TR);
    const int row0 = rb * TR + wave * RF * 16;
    const int ntf = wave * RF * 16 < nrows ? (n + 15) / 16 : 0;  // token fragments with data

    // weight rows: a uniform base per matrix and 32-bit per-lane offsets
    const uint32_t rowb = FP4 ? (uint32_t)KD / 2 : (uint32_t)KD * 2;
    const uint8_t *wbase[NMAT];
    const uint8_t *sbase[NMAT];
    uint32_t woff[RF], soff[RF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        if constexpr (FP4) {
            wbase[m] = p.wp[m] + e * p.wsp[m];
            sbase[m] = p.ws[m] + e * p.wss[m];
        } else {
            wbase[m] = reinterpret_cast<const uint8_t *>(p.wb[m]);
            sbase[m] = nullptr;
        }
    }
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        const uint32_t r = (uint32_t)min(row0 + 16 * rf + l16, rows - 1);
        woff[rf] = r * rowb + 16 * g;
        soff[rf] = r * ((uint32_t)KD / 32);
    }
    struct Chunk {
        u4 a[NMAT][RF];
        uint32_t s[NMAT][RF];
    };
    auto aload = [&](int c, Chunk &b) {
        const uint32_t cc = (uint32_t)min(c, NCH - 1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                b.a[m][rf] = *reinterpret_cast<const u4 *>(wbase[m] + (woff[rf] + cc * 64));
                if constexpr (FP4) b.s[m][rf] = *reinterpret_cast<const uint32_t *>(sbase[m] + (soff[rf] + cc * 4));
            }
    };
    // token tile: fixed per-thread source offsets (32-bit), chunk added per load
    uint32_t boff[NB];
    const uint8_t *bbase[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int v = min(tid + NT * q, NBU4 - 1);
        const int pl = v / (TOK * BSEG), vv = v - pl * (TOK * BSEG);
        const int col = vv / BSEG, seg = vv - col * BSEG;
        bbase[q] = reinterpret_cast<const uint8_t *>(p.bp[pl]);
        boff[q] = (uint32_t)bro_l[col] * (uint32_t)KD * 2 + 16 * seg;
    }
    u4 xs[NB];
    auto bload = [&](int c) {
        const uint32_t cc = (uint32_t)min(c, NCH - 1);
#pragma unroll
        for (int q = 0; q < NB; ++q) xs[q] = *reinterpret_cast<const u4 *>(bbase[q] + (boff[q] + cc * (KC * 2)));
    };
    auto bstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + NT * q;
            if (NBU4 % NT == 0 || v < NBU4) {
                const int pl = v / (TOK * BSEG), vv = v - pl * (TOK * BSEG);
                const int col = vv / BSEG, seg = vv - col * BSEG;
                *reinterpret_cast<u4 *>(B_l + buf * BBUF + (pl * TOK + col) * BROW + 16 * seg) = xs[q];
            }
        }
    };

    v4f acc[NMAT][RF][TF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
#pragma unroll
            for (int tf = 0; tf < TF; ++tf) acc[m][rf][tf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // one chunk with NTF token fragments: no branches inside
    auto compute_n = [&](const Chunk &b, int buf, auto ntf_c) {
        constexpr int NTF = decltype(ntf_c)::value;
        const uint8_t *Bb = B_l + buf * BBUF + l16 * BROW;
        float sc[NMAT][RF];
        if constexpr (FP4) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) sc[m][rf] = e8m0_to_f32((b.s[m][rf] >> (8 * g)) & 0xffu);
        }
#pragma unroll
        for (int st = 0; st < SPC; ++st) {
            bf8 a[NMAT][RF];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) {
                    if constexpr (FP4)
                        a[m][rf] = dequant8_bf16(b.a[m][rf][st], sc[m][rf]);
                    else
                        a[m][rf] = as_bf8(b.a[m][rf]);
                }
            const int kb = FP4 ? (64 * g + 16 * st) : 16 * g;  // byte offset in the token row
#pragma unroll
            for (int tf = 0; tf < NTF; ++tf) {
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl) {
                    const bf8 bv = as_bf8(*reinterpret_cast<const u4 *>(Bb + (pl * TOK + 16 * tf) * BROW + kb));
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int rf = 0; rf < RF; ++rf) acc[m][rf][tf] = mfma_bf16(a[m][rf], bv, acc[m][rf][tf]);
                }
            }
            // Schedule: each token fragment's LDS read two fragments ahead of
            // its MFMAs (left to itself the compiler reuses one register for
            // every fragment's read and waits on each read in turn)
            __builtin_amdgcn_sched_group_barrier(0x100, (NTF < 2 ? NTF : 2) * NPL, 0);
#pragma unroll
            for (int tf = 0; tf < NTF; ++tf) {
                __builtin_amdgcn_sched_group_barrier(0x008, NPL * NMAT * RF, 0);
                if (tf + 2 < NTF) __builtin_amdgcn_sched_group_barrier(0x100, NPL, 0);
            }
        }
    };
    // A chunk runs over TF, TF / 2 or TF / 4 fragments, the fewest that hold
    // the tile's tokens (a partial fragment multiplies clamped copies of the
    // last token, never stored): each is one branch-free body, so the
    // compiler keeps the accumulators in registers and overlaps the LDS reads
    // with the MFMAs (per-fragment branches serialised them); the choice is
    // one uniform branch per chunk.
    auto compute = [&](const Chunk &b, int buf) {
        if (ntf == 0) return;
        if constexpr (TF % 4 == 0) {
            if (ntf <= TF / 4) {
                compute_n(b, buf, std::integral_constant<int, TF / 4>{});
                return;
            }
        }
        if constexpr (TF % 2 == 0) {
            if (ntf <= TF / 2) {
                compute_n(b, buf, std::integral_constant<int, TF / 2>{});
                return;
            }
        }
        compute_n(b, buf, std::integral_constant<int, TF>{});
    };

    // Token loads are issued before weight loads: the LDS store of the next
    // token chunk then waits only for the token loads (memory counters retire
    // in issue order), and the weight loads stay in flight across it.
    Chunk c0, c1;
    bload(0);
    aload(0, c0);
    bstore(0);
    __syncthreads();
    for (int c = 0; c < NCH; c += 2) {
        bload(c + 1);
        aload(c + 1, c1);
        compute(c0, 0);
        bstore(1);
        __syncthreads();
        if (c + 1 >= NCH) break;
        bload(c + 2);
        aload(c + 2, c0);
        compute(c1, 1);
        bstore(0);
        __syncthreads();
    }

    tile_epilogue<KIND>(p, acc, row0, ntf, n, oro_l);
}

// A down tile on the scaled MFMA (kind kDN8): routed fp4 weights only.
// Rows and chunks as in gemm_tile; per K chunk of 128 a lane's 16 weight
// bytes (row l16, K-block g) are the A operand as loaded, its E8M0 byte the A
// scale (byte 255: the fragment is zeroed and the scale made finite, so the
// group adds exactly nothing). The token side's NPL term rows are staged
// through double-buffered LDS with one scale word per term row; a B operand
// is bytes [16g, 16g + 16) and [64 + 16g, 80 + 16g) of a term row, its scale
// byte g of the row's word.
template <int KIND>
__device__ __forceinline__ void gemm_tile_f8(const GemmParams &p, int e, int rb, int n, const int *bro_l,
                                             const int *oro_l, uint8_t *B_l)
{
    using S = GemmShape<KIND>;
    constexpr int WAVES = S::WAVES, RF = S::RF, TF = S::TF, NMAT = S::NMAT, NTB = S::NPL, TOK = S::TOK;
    constexpr int NT = 64 * WAVES;
    constexpr int KC = 128;
    constexpr int BSEG = KC / 16;                // u4 per term row per chunk
    constexpr int NBU4 = NTB * TOK * BSEG;       // u4 of one chunk's token side
    constexpr int NB = (NBU4 + NT - 1) / NT;
    constexpr int NS = NTB * TOK;                // scale words per chunk
    constexpr int NSB = (NS + NT - 1) / NT;
    constexpr int BBUF = f8_buf_bytes<KIND>();
    constexpr int SOFF = NTB * TOK * kB8Row;     // scale words after the term rows
    const int KD = p.KD, rows = p.rows, NCH = KD / KC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
    constexpr int TR = tile_rows<KIND>();
    const int nrows = min(TR, rows - rb * TR);
    const int row0 = rb * TR + wave * RF * 16;
    const int ntf = wave * RF * 16 < nrows ? (n + 15) / 16 : 0;

    const uint32_t rowb = (uint32_t)KD / 2;
    const uint8_t *wbase[NMAT];
    const uint8_t *sbase[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        wbase[m] = p.wp[m] + e * p.wsp[m];
        sbase[m] = p.ws[m] + e * p.wss[m];
    }
    uint32_t woff[RF], soff[RF];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        const uint32_t r = (uint32_t)min(row0 + 16 * rf + l16, rows - 1);
        woff[rf] = r * rowb + 16 * g;
        soff[rf] = r * ((uint32_t)KD / 32);
    }
    struct Chunk {
        u4 a[NMAT][RF];
        uint32_t s[NMAT][RF];
    };
    auto aload = [&](int c, Chunk &b) {
        const uint32_t cc = (uint32_t)min(c, NCH - 1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                b.a[m][rf] = *reinterpret_cast<const u4 *>(wbase[m] + (woff[rf] + cc * 64));
                b.s[m][rf] = *reinterpret_cast<const uint32_t *>(sbase[m] + (soff[rf] + cc * 4));
            }
    };
    // token side: fixed per-thread source offsets (32-bit), chunk added per load
    uint32_t boff[NB], toff[NSB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int v = min(tid + NT * q, NBU4 - 1);
        const int pl = v / (TOK * BSEG), vv = v - pl * (TOK * BSEG);
        const int col = vv / BSEG, seg = vv - col * BSEG;
        boff[q] = ((uint32_t)bro_l[col] * NTB + pl) * (uint32_t)KD + 16 * seg;
    }
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
        const int v = min(tid + NT * q, NS - 1);
        const int pl = v / TOK, col = v - pl * TOK;
        toff[q] = ((uint32_t)bro_l[col] * NTB + pl) * ((uint32_t)KD / 32);
    }
    u4 xs[NB];
    uint32_t xsc[NSB];
    auto bload = [&](int c) {
        const uint32_t cc = (uint32_t)min(c, NCH - 1);
#pragma unroll
        for (int q = 0; q < NB; ++q) xs[q] = *reinterpret_cast<const u4 *>(p.bq + (boff[q] + cc * KC));
#pragma unroll
        for (int q = 0; q < NSB; ++q) xsc[q] = *reinterpret_cast<const uint32_t *>(p.bsc + (toff[q] + cc * 4));
    };
    auto bstore = [&](int buf) {
        uint8_t *Bb = B_l + buf * BBUF;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + NT * q;
            if (NBU4 % NT == 0 || v < NBU4) {
                const int pl = v / (TOK * BSEG), vv = v - pl * (TOK * BSEG);
                const int col = vv / BSEG, seg = vv - col * BSEG;
                *reinterpret_cast<u4 *>(Bb + (pl * TOK + col) * kB8Row + 16 * seg) = xs[q];
            }
        }
#pragma unroll
        for (int q = 0; q < NSB; ++q) {
            const int v = tid + NT * q;
            if (NS % NT == 0 || v < NS) *reinterpret_cast<uint32_t *>(Bb + SOFF + 4 * v) = xsc[q];
        }
    };

    v4f acc[NMAT][RF][TF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
#pragma unroll
            for (int tf = 0; tf < TF; ++tf) acc[m][rf][tf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // A chunk runs over TF or TF / 2 fragments, the fewer that hold the
    // tile's tokens (as in gemm_tile; a partial fragment multiplies clamped
    // copies of the last token, never stored).
    auto compute_n = [&](const Chunk &b, int buf, auto ntf_c) {
        constexpr int NTF = decltype(ntf_c)::value;
        const uint8_t *Bb = B_l + buf * BBUF;
        v8i a[NMAT][RF];
        int sa[NMAT][RF];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                const uint32_t sbyte = (b.s[m][rf] >> (8 * g)) & 0xffu;
                const uint32_t keep = sbyte == 255u ? 0u : ~0u;
                const u4 w = b.a[m][rf];
                a[m][rf] = a_operand(u4{w.x & keep, w.y & keep, w.z & keep, w.w & keep});
                sa[m][rf] = (int)(sbyte ^ (~keep & 0x80u));   // 255 -> 127
            }
#pragma unroll
        for (int t = 0; t < NTB; ++t) {
#pragma unroll
            for (int tf = 0; tf < NTF; ++tf) {
                const int r = t * TOK + 16 * tf + l16;
                const uint8_t *row = Bb + r * kB8Row;
                const v8i bv = b_operand(*reinterpret_cast<const u4 *>(row + 16 * g),
                                         *reinterpret_cast<const u4 *>(row + 64 + 16 * g));
                const int sb = (int)((*reinterpret_cast<const uint32_t *>(Bb + SOFF + 4 * r) >> (8 * g)) & 0xffu);
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int rf = 0; rf < RF; ++rf)
                        acc[m][rf][tf] = mfma_fp4_fp8<0>(a[m][rf], bv, acc[m][rf][tf], sa[m][rf], sb);
            }
        }
        // each fragment's three LDS reads two fragments ahead of its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int f = 0; f < NTB * NTF; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x008, NMAT * RF, 0);
            if (f + 2 < NTB * NTF) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
    };
    auto compute = [&](const Chunk &b, int buf) {
        if (ntf == 0) return;
        if constexpr (TF % 2 == 0) {
            if (ntf <= TF / 2) {
                compute_n(b, buf, std::integral_constant<int, TF / 2>{});
                return;
            }
        }
        compute_n(b, buf, std::integral_constant<int, TF>{});
    };

    Chunk c0, c1;
    bload(0);
    aload(0, c0);
    bstore(0);
    __syncthreads();
    for (int c = 0; c < NCH; c += 2) {
        bload(c + 1);
        aload(c + 1, c1);
        compute(c0, 0);
        bstore(1);
        __syncthreads();
        if (c + 1 >= NCH) break;
        bload(c + 2);
        aload(c + 2, c0);
        compute(c1, 1);
        bstore(0);
        __syncthreads();
    }
    tile_epilogue<KIND>(p, acc, row0, ntf, n, oro_l);
}

// One launch: the shared expert's tiles first (bf16 weights, tokens in
// order), then the routed tiles from the list (fp4 weights).
template <int KIND>
__global__ __launch_bounds__(64 * GemmShape<KIND>::WAVES, GemmShape<KIND>::MINB) void k_gemm(GemmParams p)
{
    using S = GemmShape<KIND>;
    constexpr bool F8 = KIND == kDN8;
    constexpr bool GU = KIND != kDN && KIND != kDN8;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *B_l = lds;
    int *bro_l = reinterpret_cast<int *>(lds + gemm_tok_bytes<KIND>());  // token side row per column
    int *oro_l = bro_l + S::TOK;                                         // output row per column
    constexpr int TR = tile_rows<KIND>();
    const int RB = (p.rows + TR - 1) / TR;
    int b = blockIdx.x;
    if (!F8 && b < p.sh_blocks) {
        // the shared expert's tiles (bf16 weights p.wb, tokens in order), on
        // their own rows, reduction length, token planes and outputs
        GemmParams q = p;
        q.rows = p.sh_rows;
        q.KD = p.sh_KD;
        q.bp[0] = p.sh_bp[0];
        q.bp[1] = p.sh_bp[1];
        q.ohi = p.sh_ohi;
        q.olo = p.sh_olo;
        q.oq = nullptr;
        q.osc = nullptr;
        const int RBs = (q.rows + TR - 1) / TR;
        const int tile = b / RBs, rb = b - tile * RBs;
        const int p0 = tile * S::TOK, n = min(S::TOK, p.T - p0);
        for (int c = threadIdx.x; c < S::TOK; c += 64 * S::WAVES) {
            const int t = p0 + min(c, n - 1);
            bro_l[c] = t;
            oro_l[c] = GU ? t : t * (p.K + 1) + p.K;
        }
        __syncthreads();
        if constexpr (!F8) gemm_tile<KIND, false>(q, 0, rb, p0, n, bro_l, oro_l, B_l);
        return;
    }
    b -= p.sh_blocks;
    const int tile = b / RB, rb = b - tile * RB;
    if (tile >= *p.tile_n) return;
    const int2 tl = p.tiles[tile];
    const int e = p.active_e[tl.x];
    const int p0 = p.active_off[tl.x] + tl.y * S::TOK, n = min(S::TOK, p.active_off[tl.x + 1] - p0);
    for (int c = threadIdx.x; c < S::TOK; c += 64 * S::WAVES) {
        const int cc = min(c, n - 1);
        const int a = p.sorted[p0 + cc];
        bro_l[c] = GU ? a / p.K : p0 + cc;
        oro_l[c] = GU ? p0 + cc : (a / p.K) * (p.K + 1) + a % p.K;
    }
    __syncthreads();
    if constexpr (F8)
        gemm_tile_f8<KIND>(p, e, rb, n, bro_l, oro_l, B_l);
    else
        gemm_tile<KIND, true>(p, e, rb, p0, n, bro_l, oro_l, B_l);
}

}  // namespace

// Launch-time limits of the grouped kernels (hidden, inter, shared inter are
// validated multiples of 128 at layer creation).
static bool set_lds_limits()
{
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<kGU>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gemm_lds_bytes<kGU>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<kDN>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gemm_lds_bytes<kDN>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<kGU2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gemm_lds_bytes<kGU2>());
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<kDN8>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, gemm_lds_bytes<kDN8>());
    return true;
}

// Upper bound on the tiles of bn tokens: every expert with more than smax
// assignments (smax: the light-expert limit of the streaming kernels, 0 when
// they are off) adds at most one partial tile, and there are at most
// min(E, T*K / (smax + 1)) such experts.
size_t grouped_tile_cap(int64_t T, int K, int E, int bn, int smax)
{
    const int64_t n = T * K;
    return (size_t)(n / bn + std::min<int64_t>(E, n / (smax + 1)) + 1);
}

// Workspace sizes: the smaller gate/up tile of the two token forms
size_t grouped_tile_cap_gu(int64_t T, int K, int E)
{
    return grouped_tile_cap(T, K, E, std::min(GemmShape<kGU>::TOK, GemmShape<kGU2>::TOK), 0);
}
size_t grouped_tile_cap_dn(int64_t T, int K, int E) { return grouped_tile_cap(T, K, E, GemmShape<kDN>::TOK, 0); }

hipError_t launch_grouped(const LayerView &L, const uint16_t *x, const uint16_t *xr, const uint16_t *xr_lo, int T,
                          const int32_t *active_n, const int32_t *active_e, const int32_t *active_off,
                          const int32_t *sorted, uint16_t *act_hi, uint16_t *act_lo, uint16_t *ash_hi,
                          uint16_t *ash_lo, float *sh_part, int2 *tiles_gu, int2 *tiles_dn, int32_t *light,
                          int32_t *counts, float *ys, float *ysh, hipStream_t s, Profiler *prof,
                          const TermBufs &tb)
{
    static const bool lds_set = set_lds_limits();  // once per process (thread-safe static)
    (void)lds_set;
    const bool two = xr_lo != nullptr;  // routed tokens as hi and lo planes
    const int TG = two ? GemmShape<kGU2>::TOK : GemmShape<kGU>::TOK, TD = GemmShape<kDN>::TOK;
    constexpr int TGS = GemmShape<kGU>::TOK;  // the shared expert's gate/up tiles
    auto blocks = [](int rows, int tr) { return (rows + tr - 1) / tr; };
    const int rb_i = blocks(L.I, tile_rows<kGU>());    // gate/up rows (every gate/up kind: the same rows per block)
    const int rb_h = blocks(L.H, tile_rows<kDN>());    // the shared expert's down rows
    const int rb_r = blocks(L.EK, tile_rows<kDN>());   // routed down rows (every down kind)
    const int rb_s = blocks(L.Is, tile_rows<kGU>());   // the shared expert's gate/up rows
    const bool stream = stream_path_ok(L), stream_dn = stream_down_ok(L, T);
    const bool sh_stream = stream_shared_ok(L, T);
    const int smax_gu = stream ? stream_max_tokens() : 0, smax_dn = stream_dn ? stream_down_rows(L, T) : 0;
    // grids cover the most tiles the split can produce (most blocks exit at once)
    const size_t cap_gu = grouped_tile_cap(T, L.K, L.E, TG, smax_gu), cap_dn = grouped_tile_cap(T, L.K, L.E, TD, smax_dn);
    int32_t *light_gu = light, *light_dn = light + L.E, *light1 = light + 2 * L.E, *light2 = light + 3 * L.E;
    // no expert can hold more than T * K assignments (T when the ids come
    // from the router: no expert twice in a token): when that fits the
    // streamed limit, no tile is heavy and the tile GEMMs would only exit
    const int64_t most = L.routes_distinct ? (int64_t)T : (int64_t)T * L.K;
    const bool gemm_gu = !(stream && most <= smax_gu), gemm_dn = !(stream_dn && most <= smax_dn);
    // the scaled-MFMA down tiles: when every expert on down tiles also ran
    // gate/up on tiles (smax_dn >= smax_gu), whose epilogue then writes the
    // activation's terms; it also writes hi/lo when the streamed down
    // projection reads rows of experts that ran gate/up on tiles
    const bool f8_dn = gemm_dn && gemm_gu && smax_dn >= smax_gu && tb.aq != nullptr;
    const bool hilo_from_tiles = !f8_dn || smax_dn > smax_gu;
    // light experts with one or two assignments (a flat layer) stream their
    // gate/up rows through the one-token kernel's whole-piece loads
    const bool one_gu = stream && !two && gu_one_ok(L);
    k_tiles<<<1, 1024, 0, s>>>(active_n, active_off, TG, TD, smax_gu, smax_dn, one_gu ? 1 : 0, tiles_gu, tiles_dn,
                               light_gu, light_dn, light1, light2, counts);

    // gate/up: routed tiles (fp4); the shared expert's tiles go in a launch of
    // their own (different weight rows) unless they stream with the light experts
    {
        StageMark m(prof, K3MOE_STAGE_GATEUP, s);
        if (stream) {
            const hipError_t e = launch_stream_gu(L, x, xr, xr_lo, T, active_e, active_off, sorted, light_gu,
                                                  counts + 2, sh_stream, act_hi, act_lo, ash_hi, ash_lo, sh_part, s);
            if (e != hipSuccess) return e;
        }
        for (int nt = 1; one_gu && nt <= 2; ++nt) {
            const hipError_t e = launch_gu_one(L, xr, T, nt, active_e, active_off, sorted, nt == 1 ? light1 : light2,
                                               counts + 3 + nt, act_hi, act_lo, s);
            if (e != hipSuccess) return e;
        }
        GemmParams gp{};
        gp.rows = L.I;
        gp.KD = L.EK;
        gp.K = L.K;
        gp.T = T;
        gp.act = L.act;
        gp.b1 = L.b1;
        gp.b2 = L.b2;
        gp.wp[0] = L.gp;
        gp.wp[1] = L.up;
        gp.ws[0] = L.gs;
        gp.ws[1] = L.us;
        gp.wsp[0] = L.g_sp;
        gp.wsp[1] = L.u_sp;
        gp.wss[0] = L.g_ss;
        gp.wss[1] = L.u_ss;
        gp.bp[0] = xr;
        gp.bp[1] = two ? xr_lo : xr;
        gp.active_e = active_e;
        gp.active_off = active_off;
        gp.sorted = sorted;
        gp.tiles = tiles_gu;
        gp.tile_n = counts;
        gp.ohi = hilo_from_tiles ? act_hi : nullptr;
        gp.olo = hilo_from_tiles ? act_lo : nullptr;
        gp.oq = f8_dn ? tb.aq : nullptr;
        gp.osc = f8_dn ? tb.aqs : nullptr;
        // the shared expert's gate/up tiles: in the routed tiles' launch when
        // both are one bf16 token plane (its long blocks first in the grid,
        // beside the routed ones), else in a launch of their own
        const bool sh_tiles = L.Is > 0 && !sh_stream;
        const bool sh_merged = sh_tiles && gemm_gu && !two;
        if (sh_tiles) {
            gp.wb[0] = L.sh_gate;
            gp.wb[1] = L.sh_up;
            gp.sh_rows = L.Is;
            gp.sh_KD = L.H;
            gp.sh_bp[0] = gp.sh_bp[1] = x;
            gp.sh_ohi = ash_hi;
            gp.sh_olo = ash_lo;
        }
        const int sh_blocks = sh_tiles ? ((T + TGS - 1) / TGS) * rb_s : 0;
        if (gemm_gu) {
            StageMark mt(prof, K3MOE_STAGE_GATEUP_TILES, s);
            if (two) {
                k_gemm<kGU2><<<(unsigned)(cap_gu * rb_i), 64 * GemmShape<kGU2>::WAVES, gemm_lds_bytes<kGU2>(), s>>>(gp);
            } else {
                gp.sh_blocks = sh_merged ? sh_blocks : 0;
                k_gemm<kGU><<<(unsigned)(gp.sh_blocks + cap_gu * rb_i), 64 * GemmShape<kGU>::WAVES,
                               gemm_lds_bytes<kGU>(), s>>>(gp);
            }
        }
        if (sh_tiles && !sh_merged) {
            StageMark m2(prof, K3MOE_STAGE_SHARED_GATEUP, s);
            GemmParams sp = gp;
            sp.sh_blocks = sh_blocks;
            k_gemm<kGU><<<(unsigned)sp.sh_blocks, 64 * GemmShape<kGU>::WAVES, gemm_lds_bytes<kGU>(), s>>>(sp);
        }
    }
    {
        StageMark m(prof, K3MOE_STAGE_DOWN, s);
        if (stream_dn) {
            const hipError_t e = launch_stream_dn(L, T, active_e, active_off, sorted, light_dn, counts + 3,
                                                  sh_stream, act_hi, act_lo, ash_hi, ash_lo, ys, ysh, s);
            if (e != hipSuccess) return e;
        }
        GemmParams dp{};
        dp.rows = L.EK;
        dp.KD = L.I;
        dp.K = L.K;
        dp.T = T;
        dp.wp[0] = dp.wp[1] = L.dp;
        dp.ws[0] = dp.ws[1] = L.ds;
        dp.wsp[0] = dp.wsp[1] = L.d_sp;
        dp.wss[0] = dp.wss[1] = L.d_ss;
        dp.bp[0] = act_hi;
        dp.bp[1] = act_lo;
        dp.active_e = active_e;
        dp.active_off = active_off;
        dp.sorted = sorted;
        dp.tiles = tiles_dn;
        dp.tile_n = counts + 1;
        dp.ys = ys;
        if (gemm_dn) {
            StageMark mt(prof, K3MOE_STAGE_DOWN_TILES, s);
            if (f8_dn) {
                GemmParams fp = dp;
                fp.bq = tb.aq;
                fp.bsc = tb.aqs;
                k_gemm<kDN8><<<(unsigned)(cap_dn * rb_r), 64 * GemmShape<kDN8>::WAVES, gemm_lds_bytes<kDN8>(), s>>>(fp);
            } else {
                k_gemm<kDN><<<(unsigned)(cap_dn * rb_r), 64 * GemmShape<kDN>::WAVES, gemm_lds_bytes<kDN>(), s>>>(dp);
            }
        }
        if (L.Is > 0 && !sh_stream) {
            // shared rows of H: to slot k of ys (flat), or to ysh [T][H] (K = 0 makes the row t)
            GemmParams sp = dp;
            sp.sh_rows = L.H;
            sp.sh_KD = L.Is;
            sp.K = ysh ? 0 : L.K;
            sp.ys = ysh ? ysh : ys;
            sp.wb[0] = sp.wb[1] = L.sh_down;
            sp.sh_bp[0] = ash_hi;
            sp.sh_bp[1] = ash_lo;
            sp.sh_blocks = ((T + TD - 1) / TD) * rb_h;
            k_gemm<kDN><<<(unsigned)sp.sh_blocks, 64 * GemmShape<kDN>::WAVES, gemm_lds_bytes<kDN>(), s>>>(sp);
        }
    }
    return hipGetLastError();
}

}  // namespace k3moe
