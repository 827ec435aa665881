// The one-token layer of a flat layer in three launches: route + experts +
// router-order combine ("kimi-k3-in-c" README §9 "Picking 16 experts of
// 896": k3_router, k3_moe steps 3 and 6, k3_situ_glu; §4 "Reduction one: the
// experts already ship at half a byte": the MXFP4 format).
//
//   R  (k_router)            the router rows (logits, scores)
//   G  (k_dec_gateup)        the top-k, the routed experts' gate/up rows
//                            and activations (written as e4m3 terms), and
//                            an equal share of the shared expert's rows in
//                            every block
//   D  (k_dec_down)          the shared expert's down rows, the routed
//                            experts' down rows, the router-order weighted
//                            sum, the output
//
// Decode is a stream of weights from HBM: the design aims at the access
// pattern a plain streaming read runs fastest with on MI355X, one wave
// instruction = one contiguous kilobyte of one weight row, and at as few
// launches as the data dependencies allow (route -> gate/up -> down).
//
// MFMA with row-contiguous loads. A wave's 64 lanes hold 64 consecutive
// 16-byte pieces of ONE weight row (one 32-weight group each), not the
// 16 rows x 64 bytes the MFMA operand layout asks for. The MFMA still does
// the dot products: each lane also holds, as its B fragment, the other
// operand at the same K positions as its own A fragment, so the product of a
// lane's A with its own B sits on the diagonal of the 16 x 16 result
// (C[i][i] sums lanes i, i+16, i+32, i+48), and the row's dot product is
// the sum of the diagonal. Off-diagonal entries are never read.
//  * bf16 MFMA (v_mfma_f32_16x16x32_bf16, gate/up): A and B take the same K
//    positions in the same lane, so a lane's B is simply the token at its
//    weights' positions, kept in registers for every row.
//  * Scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, down): the fp4 A of
//    lane (i, g) = lane i + 16 g is the 32 K positions [32g, 32g + 32) of
//    MFMA row i, while the fp8 B of lane (i, g') holds K positions
//    [16g', 16g' + 16) in bytes 0..15 and [64 + 16g', 80 + 16g') in bytes
//    16..31 of column i. So lane (i, g') loads, for its B, half g' & 1 of
//    the activation pieces that lanes (i, g'/2) and (i, 2 + g'/2) multiply;
//    the scale of B's K-block g comes from lane (i, g), which holds exactly
//    that block's term scale.
#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

// e4m3 terms of a routed activation: three leave about 2^-14 of each
// 32-element block's maximum out
constexpr int kDecTerms = 3;

// Loads in the streaming loops are plain loads from clamped (always valid)
// addresses: a lane past a row's end reads real weights that meet a zero
// operand on the other side (or a zero scale), so nothing is masked after
// the load. Operands that stay in registers (the token, the activations, the
// e4m3 terms) are masked once, when they are loaded, with a mask the
// compiler cannot see through: a select on a loaded value may otherwise be
// turned into a branch around the load, and a branch around a load makes the
// wait-count pass drain every load in flight at the join.
__device__ __forceinline__ uint32_t lane_mask(bool on)
{
    uint32_t m = on ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));
    return m;
}
__device__ __forceinline__ u4 ld16m(const void *p, uint32_t m)
{
    const u4 v = *reinterpret_cast<const u4 *>(p);
    return u4{v.x & m, v.y & m, v.z & m, v.w & m};
}

// Sum over the wave, fixed order, through DPP (quad steps, half-row and row
// mirrors, then the row broadcasts into lane 63), read back from lane 63.
__device__ __forceinline__ float wave_sum(float v)
{
#define K3_DPP(x, ctrl, rmask) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xf, false))
    v += K3_DPP(v, 0xb1, 0xf);   // quad [1,0,3,2]
    v += K3_DPP(v, 0x4e, 0xf);   // quad [2,3,0,1]
    v += K3_DPP(v, 0x141, 0xf);  // row_half_mirror
    v += K3_DPP(v, 0x140, 0xf);  // row_mirror
    v += K3_DPP(v, 0x142, 0xa);  // row_bcast15 into rows 1, 3
    v += K3_DPP(v, 0x143, 0xc);  // row_bcast31 into rows 2, 3
#undef K3_DPP
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}


// Diagonal of a 16 x 16 MFMA result, summed: lane L holds
// C[4 (L / 16) + r][L % 16] in acc[r], so C[i][i] sits in the lanes with
// (L % 16) / 4 == L / 16, register L % 4.
__device__ __forceinline__ float diag_sum(const v4f acc)
{
    const int L = threadIdx.x & 63, r = L & 3;
    const float v = r == 0 ? acc[0] : r == 1 ? acc[1] : r == 2 ? acc[2] : acc[3];
    return wave_sum((((L & 15) >> 2) == (L >> 4)) ? v : 0.0f);
}

// The diagonals of four 16 x 16 MFMA results, summed together (lane L holds
// C[4 (L / 16) + r][L % 16] in acc[k][r]; the diagonal entries sit in the
// lanes with (L % 16) / 4 == L / 16, register L % 4). Every lane keeps its
// diagonal value of each result (0 elsewhere); an exchange with lane L ^ 32
// leaves lanes 0..31 the partial sums of results 0 and 1 and lanes 32..63
// those of 2 and 3, an exchange with lane L ^ 16 leaves lane group L / 16
// with result L / 16 alone, and four DPP steps sum each 16-lane group: every
// lane of group k returns result k. The same sums as four separate wave
// sums, in another order, with a quarter of the cross-lane steps.
__device__ __forceinline__ float diag_sum4(const v4f (&acc)[4])
{
    const int L = threadIdx.x & 63, r = L & 3;
    const bool dg = ((L & 15) >> 2) == (L >> 4);
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float e = r == 0 ? acc[k][0] : r == 1 ? acc[k][1] : r == 2 ? acc[k][2] : acc[k][3];
        v[k] = dg ? e : 0.0f;
    }
    const bool hi = L >= 32;
    const float g0 = __shfl_xor(hi ? v[0] : v[2], 32), g1 = __shfl_xor(hi ? v[1] : v[3], 32);
    const float a0 = (hi ? v[2] : v[0]) + g0, a1 = (hi ? v[3] : v[1]) + g1;
    const bool b4 = (L & 16) != 0;
    float w = (b4 ? a1 : a0) + __shfl_xor(b4 ? a0 : a1, 16);
#define K3_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false))
    w += K3_DPP(w, 0xb1);   // quad [1,0,3,2]
    w += K3_DPP(w, 0x4e);   // quad [2,3,0,1]
    w += K3_DPP(w, 0x141);  // row_half_mirror
    w += K3_DPP(w, 0x140);  // row_mirror
#undef K3_DPP
    return w;
}

// ---------------------------------------------------------------------------
// G: the routed experts' gate/up rows, one E8M0 block of a slot's activation
// per 4-wave block: block q of slot j takes rows [32 q', 32 q' + 32) of gate
// and up (q' = q mod I/32), and an equal share of the shared expert's row
// pairs (pairs [Is q / NB, Is (q + 1) / NB) of the NB = K I / 32 blocks), so
// every block streams the same bytes and the grid is one even round of
// blocks (768 of 280 KB at the full shape, three per CU). Wave w streams ONE
// matrix (w & 1: gate, up) over 16 routed rows (w >> 1: the first or second
// half), one weight stream per wave: on MI355X a wave with one contiguous
// stream and two rows in flight keeps HBM busier than one interleaving two
// streams. Each wave
//  1. wave 0 issues the loads of the router's scores; after a block barrier
//     (issue order: the scores ahead of the shared rows' burst) waves 1..3
//     issue the loads of their first shared row (row t = w, w + 4, ... of
//     the block's 2P rows, gate and up of pair t / 2 alternating) while wave
//     0 takes the top-k (or reads the given ids);
//  2. after the block barrier that publishes the expert id, each wave issues
//     its first two routed rows, its 16 E8M0 rows and its share of the
//     token (wave 0 then its shared row), and stores the token and the E8M0
//     rows to LDS;
//  3. after a block barrier, finishes its shared rows (bf16 x bf16 fp32 FMA
//     in slice order, one wave-wide sum each, parked in LDS);
//  4. takes the token from LDS into registers at its lanes' K positions
//     (lane l of row piece s: elements 2048 s + 32 l + [0, 32)) and streams
//     its 16 routed rows, two in flight, each row piece as 4 bf16 MFMAs
//     after an exact fp4 -> bf16 expansion (the diagonal dot product);
//  5. parks its 16 sums in LDS; after the block barrier wave 0 takes the 32
//     routed activations and splits them into kDecTerms e4m3 terms with one
//     E8M0 scale per term (the form the down kernel's scaled MFMA takes), and
//     wave 1 writes the block's shared activations.
constexpr int kDecGuPieces = 4;    // 1 KB pieces per row: H <= 8192
constexpr int kDecUnitRows = 16;   // rows per wave
constexpr int kDecShPairs = 64;    // shared row pairs per block, at most

struct DecGuParams {
    const uint8_t *gp, *gs, *up, *us;
    int64_t g_sp, g_ss, u_sp, u_ss;
    int H, I, E, K, act;
    float b1, b2;
    int renorm;
    float rscale;
    const uint16_t *x;          // bf16 [H]
    const float *sc, *ch;       // router scores [E] (fused top-k)
    int32_t *idx;               // [K]: written by block 0 (fused top-k) or read
    float *w;                   // [K]: written by block 0 (fused top-k)
    uint8_t *aq;                // e4m3 terms [K][kATerms][I] (the first kDecTerms written)
    uint8_t *as;                // their E8M0 scales [K][kATerms][I / 32]
    const uint16_t *sh_gate, *sh_up;  // bf16 [Is][H]
    float *ash;                 // [Is] out: the shared expert's activation
    int Is;
};

// LDS: the 4 waves' E8M0 rows (16 x H/32 bytes each), the top-k scratch,
// the expert id, the parked routed sums [4][16], the shared rows' sums
// [2 kDecShPairs], the token as bf16 slices [NS][64] u4.
__host__ __device__ constexpr int dec_gu_lds_bytes(int H, int NS)
{
    return 4 * (H / 2) + (int)sizeof(TopkLds) + 16 + 4 * 16 * 4 + 2 * kDecShPairs * 4 + NS * 64 * 16;
}

// Split the activations held by lanes 0..31 (one E8M0 block) into kDecTerms
// e4m3 terms: per term, the scale puts the block's largest remainder in
// [224, 448], the term takes only the elements within 6 binades of that
// maximum (the scaled MFMA sums 16-product runs to about 14 bits below the
// run's largest product) and its rounding error is carried exactly into the
// next term.
__device__ __forceinline__ void split_terms_32(float r, uint8_t *term, size_t term_stride, uint8_t *sc,
                                               size_t sc_stride)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < kDecTerms; ++t) {
        float m = fabsf(r);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));  // within lanes 0..31
        int S = 0;
        float keep_min = INFINITY;
        if (m > 0.0f) {
            int ex;
            frexpf(m, &ex);
            S = ex - 9;
            if (ldexpf(m, -S) > 448.0f) S += 1;
            if (S < -127) S = -127;
            frexpf(ldexpf(m, -S), &ex);
            keep_min = ldexpf(1.0f, ex - 7);
        }
        const float q = ldexpf(r, -S);
        uint32_t c = 0;
        if (fabsf(q) >= keep_min) {
            c = __builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xffu;
            r -= ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)c, 0), S);
        }
        if (lane < 32) term[t * term_stride + lane] = (uint8_t)c;
        if (lane == 0) sc[t * sc_stride] = (uint8_t)(S + 127);
    }
}

// NQ > 0: wave 0 takes the top-k here (16-byte score loads, NQ experts per
// lane); NQ == 0: the ids are read from p.idx. NS: 512-element slices of a
// shared row (H <= 512 NS).
template <int NQ, int NS>
__global__ __launch_bounds__(256, 3) void k_dec_gateup(DecGuParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int bid = blockIdx.x, nb = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = p.H, HB = H >> 1, HG = H >> 5;  // packed bytes and E8M0 groups per row
    const int NG = p.I >> 5;                      // E8M0 blocks per slot activation
    const int j = bid / NG, qb = bid - j * NG;
    const int mat = wave & 1, half = wave >> 1;
    uint8_t *sc_l = lds + wave * (H / 2);
    TopkLds &tl = *reinterpret_cast<TopkLds *>(lds + 2 * H);
    int *e_l = reinterpret_cast<int *>(lds + 2 * H + sizeof(TopkLds));
    float *sum_l = reinterpret_cast<float *>(lds + 2 * H + sizeof(TopkLds) + 16);  // [4][16]
    float *shs_l = sum_l + 4 * kDecUnitRows;                                      // [2 kDecShPairs]
    u4 *x_l = reinterpret_cast<u4 *>(shs_l + 2 * kDecShPairs);                    // [NS][64]

    // 1. wave 0 issues the router scores' loads; the block barrier then
    // orders them ahead of every shared row's load
    constexpr int NQL = NQ > 0 ? NQ : 1;
    float raw[NQL], sv[NQL];
    if constexpr (NQ > 0)
        if (wave == 0) topk_load<NQ, true>(p.sc, p.ch, p.E, raw, sv);
    __syncthreads();  // issue order only

    // 2. this block's shared rows: pairs [sp0, sp1), row t = pair sp0 + t/2 of
    // gate (t even) or up (t odd); wave w takes rows w, w + 4, ...; waves
    // 1..3 issue their first row's loads now, wave 0 takes the top-k (no
    // memory access but the scores) and loads its shared row later
    const int sp0 = (int)((int64_t)p.Is * bid / nb), sp1 = (int)((int64_t)p.Is * (bid + 1) / nb);
    const int nsr = 2 * (sp1 - sp0);
    auto sh_row = [&](int t) {
        const int n = sp0 + (t >> 1);
        return ((t & 1) ? p.sh_up : p.sh_gate) + (size_t)n * H;
    };
    u4 shw[NS];
    auto sh_load = [&](int t) {
        const uint16_t *r = sh_row(t < nsr ? t : 0);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int i = 512 * s + 8 * lane;
            shw[s] = ld16_stream(r + (i < H ? i : 0));  // off lanes meet a zero token
        }
    };
    if (wave != 0 && wave < nsr) sh_load(wave);
    if constexpr (NQ > 0) {
        if (wave == 0) {
            int pick;
            float wt;
            topk_rank<NQ>(raw, sv, p.E, p.K, p.renorm, p.rscale, tl, &pick, &wt);
            if (bid == 0 && lane < p.K) {
                p.idx[lane] = pick;
                p.w[lane] = wt;
            }
            if (lane == 0) e_l[0] = __builtin_amdgcn_readlane(pick, j);
        }
    } else {
        if (threadIdx.x == 0) e_l[0] = p.idx[j];
    }
    __syncthreads();  // the expert id

    int e = e_l[0];
    const bool ok = e >= 0 && e < p.E;  // an invalid id: zero activations (the down kernel drops it)
    e = ok ? e : 0;

    // 3. the routed rows' first loads, this wave's 16 E8M0 rows (contiguous:
    // 16 x H/32 bytes) and the token (u4 i: elements 8i .. 8i + 7, zero past
    // H); wave 0's shared row last
    const int row0 = 32 * qb + kDecUnitRows * half;
    const uint8_t *sbase = (mat ? p.us + (int64_t)e * p.u_ss : p.gs + (int64_t)e * p.g_ss) + (size_t)row0 * HG;
    const uint8_t *wbase = (mat ? p.up + (int64_t)e * p.u_sp : p.gp + (int64_t)e * p.g_sp) + (size_t)row0 * HB;
    int soff[kDecGuPieces];        // this lane's offset in a row piece (off lanes: the last on lane's)
    int gidx[kDecGuPieces];        // this lane's E8M0 group (off lanes: 0)
    uint32_t smask[kDecGuPieces];  // off lanes scale their weights by 0
#pragma unroll
    for (int s = 0; s < kDecGuPieces; ++s) {
        const bool on = 64 * s + lane < HG;
        // an off lane repeats the last on lane's address (in the same
        // instruction when the piece has on lanes, so no line is fetched
        // twice: the streaming loads leave nothing in the caches to re-read)
        soff[s] = min(1024 * s + 16 * lane, HB - 16);
        gidx[s] = on ? 64 * s + lane : 0;
        smask[s] = lane_mask(on);
    }
    struct Row {
        u4 a[kDecGuPieces];
    };
    auto load = [&](int r, Row &b) {
        const size_t ro = (size_t)min(r, kDecUnitRows - 1) * HB;
#pragma unroll
        for (int s = 0; s < kDecGuPieces; ++s) b.a[s] = ld16_stream(wbase + ro + soff[s]);
    };
    constexpr int GD = 2;  // rows in flight (four measured slower)
    Row bq[GD];
#pragma unroll
    for (int d = 0; d < GD; ++d) load(d, bq[d]);
    constexpr int SQ = 8192 / 2 / 1024;  // 16-byte pieces per lane (H <= 8192)
    u4 scv[SQ];
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        const int i = 16 * lane + 1024 * k;
        scv[k] = ld16_stream(sbase + min(i, H / 2 - 16));  // off lanes: the last on lane's address
    }
    constexpr int XQ = (NS * 64 + 255) / 256;
    {
        u4 xs[XQ];
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int i = threadIdx.x + 256 * q;
            const bool on = i < NS * 64 && 8 * i < H;
            xs[q] = ld16m(p.x + (on ? 8 * i : 0), lane_mask(on));
        }
        if (wave == 0 && nsr > 0) sh_load(0);
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int i = threadIdx.x + 256 * q;
            if (i < NS * 64) x_l[i] = xs[q];
        }
    }
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        const int i = 16 * lane + 1024 * k;
        if (i < H / 2) *reinterpret_cast<u4 *>(sc_l + i) = scv[k];
    }
    __syncthreads();  // the token slices (and this wave's E8M0 rows)

    // 3. the shared rows
    for (int t = wave; t < nsr; t += 4) {
        if (t != wave) sh_load(t);
        float a = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u4 xq = x_l[s * 64 + lane];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a = fmaf(bf16f(shw[s][q] & 0xffffu), bf16f(xq[q] & 0xffffu), a);
                a = fmaf(bf16f(shw[s][q] >> 16), bf16f(xq[q] >> 16), a);
            }
        }
        a = wave_sum(a);
        if (lane == 0) shs_l[t] = a;
    }

    // 4. the token at this lane's K positions (lane l of row piece s:
    // elements 2048 s + 32 l + [0, 32)), from LDS
    u4 xv[kDecGuPieces][4];
#pragma unroll
    for (int s = 0; s < kDecGuPieces; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = 2048 * s + 32 * lane + 8 * c;
            xv[s][c] = ld16m(x_l + (i < H ? i / 8 : 0), lane_mask(i < H));
        }

    float mine = 0.0f;
    auto compute = [&](int r, const Row &b) {
        v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kDecGuPieces; ++s) {
            const float f = __uint_as_float(__float_as_uint(e8m0_to_f32(sc_l[r * HG + gidx[s]])) & smask[s]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc = mfma_bf16(dequant8_bf16(b.a[s][c], f), as_bf8(xv[s][c]), acc);
        }
        const float v = diag_sum(acc);
        mine = lane == r ? v : mine;
    };
    // fully unrolled: the rows' next loads stop at the last row (a load past
    // it would re-read a row the streaming loads have not kept)
#pragma unroll
    for (int r = 0; r < kDecUnitRows; r += GD) {
        prio_left(kDecUnitRows - r, kDecUnitRows);
#pragma unroll
        for (int d = 0; d < GD; ++d) {
            compute(r + d, bq[d]);
            if (r + d + GD < kDecUnitRows) load(r + d + GD, bq[d]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (lane < kDecUnitRows) sum_l[wave * kDecUnitRows + lane] = mine;
    __syncthreads();

    // 5. wave 0: the 32 activations (lane l: row 32 qb + l) as e4m3 terms;
    // wave 1: the block's shared activations
    if (wave == 0) {
        const int hl = (lane >> 4) & 1, rl = lane & 15;  // lanes 32..63 repeat 0..31 (unused)
        const float g = sum_l[(2 * hl) * kDecUnitRows + rl], u = sum_l[(2 * hl + 1) * kDecUnitRows + rl];
        const float a = ok ? act_fn(g, u, p.act, p.b1, p.b2) : 0.0f;
        split_terms_32(lane < 32 ? a : 0.0f, p.aq + ((size_t)j * kATerms) * p.I + (size_t)qb * 32, p.I,
                       p.as + ((size_t)j * kATerms) * NG + qb, NG);
    } else if (wave == 1 && 2 * lane < nsr) {
        p.ash[sp0 + lane] = act_fn(shs_l[2 * lane], shs_l[2 * lane + 1], p.act, p.b1, p.b2);
    }
}

// ---------------------------------------------------------------------------
// D: the routed experts' down rows, the shared expert's down rows and the
// router-order sum. Block b owns output rows [b RB, b RB + RB) for every
// slot; wave w takes slot w. A slot's B operands (kDecTerms e4m3 terms of its
// activation, arranged for the diagonal) and their scales stay in registers
// for all the block's rows; a row of W2 is one wave instruction (lane l:
// group l, I/32 lanes), kDecDnDepth rows in flight. The shared expert's rows
// of the block (wave w: rows w and w + NW) are loaded first, while the routes
// are read, and multiplied after the routed rows. The per-slot results go to
// LDS and one pass sums them in router order, adds the shared row and
// applies the epilogue. Every load before the routed loop is unconditional
// (clamped addresses, a compile-time slice count, the routing weights and
// the shared activation held in registers and written to LDS after the
// loop), so the compiler's wait counts keep the rows in flight instead of
// draining them at a branch.
constexpr int kDecDnWaves = 16;            // one slot per wave
constexpr int kDecDnDepth = 4;             // rows in flight per wave (diag_sum4 takes four)
constexpr int kDecDnRowsMax = 32;          // rows a block owns, at most
constexpr int kDecShRows = kDecDnRowsMax / kDecDnWaves;  // shared rows per wave

struct DecDnParams {
    const uint8_t *dp, *ds;
    int64_t d_sp, d_ss;
    int H, I, E, K, RB;
    const int32_t *idx;
    const float *w;
    const uint8_t *aq, *as;
    const uint16_t *sh_down;    // bf16 [H][Is] (Is == 0: none)
    const float *ash;           // [Is]
    int Is;
    float *out;
    int resid;
    uint16_t *ob;
    unsigned long long *errors;
};

// NSS: 512-element slices of a shared row, ceil(I_s / 512) <= 4 (0: no
// shared expert)
template <int NSS>
__global__ __launch_bounds__(64 * kDecDnWaves) void k_dec_down(DecDnParams p)
{
    extern __shared__ __align__(16) float y_l[];  // [K][RB], then (16-byte aligned) the shared activation [Is]
    __shared__ float wk_l[kMaxTopk];  // routing weights, 0 for an id outside [0, E)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int I = p.I, NG = I >> 5, IB = I >> 1;
    const int r0 = blockIdx.x * p.RB, nr = min(p.RB, p.H - r0);
    const bool has = wave < p.K;  // this wave's slot exists (else it computes slot 0 and drops it)
    const int jj = has ? wave : 0;
    const bool on = lane < NG;

    // the slot's B operands: the e4m3 terms arranged for the diagonal (the
    // first loads, so that using them waits for nothing else)
    v8i bt[kDecTerms];
    int bs[kDecTerms];
    {
        const int i16 = lane & 15, g4 = lane >> 4;
        const int p0 = 32 * (i16 + 16 * (g4 >> 1)) + 16 * (g4 & 1);
        const int p1 = 32 * (i16 + 16 * (2 + (g4 >> 1))) + 16 * (g4 & 1);
#pragma unroll
        for (int t = 0; t < kDecTerms; ++t) {
            const uint8_t *tr = p.aq + ((size_t)jj * kATerms + t) * I;
            const u4 l2 = ld16m(tr + (p0 < I ? p0 : 0), lane_mask(p0 < I));
            const u4 h2 = ld16m(tr + (p1 < I ? p1 : 0), lane_mask(p1 < I));
            bt[t] = v8i{(int)l2.x, (int)l2.y, (int)l2.z, (int)l2.w, (int)h2.x, (int)h2.y, (int)h2.z, (int)h2.w};
            bs[t] = on ? (int)p.as[((size_t)jj * kATerms + t) * NG + lane] : 127;
        }
    }

    const int e0 = p.idx[jj];

    // the shared expert's rows of this block: wave w takes rows r0 + w + NW k,
    // issued before the wait for the expert id (the barrier keeps them there)
    __shared__ float sh_l[kDecDnRowsMax];
    float *ash_l = y_l + ((p.K * p.RB + 3) & ~3);  // 16-byte aligned
    u4 shw[kDecShRows][NSS > 0 ? NSS : 1];
    if constexpr (NSS > 0) {
#pragma unroll
        for (int k = 0; k < kDecShRows; ++k) {
            const int r = r0 + min(wave + kDecDnWaves * k, nr - 1);
#pragma unroll
            for (int sl = 0; sl < NSS; ++sl) {
                const bool son = 512 * sl + 8 * lane < p.Is;
                shw[k][sl] = ld16_stream(p.sh_down + (size_t)r * p.Is + (son ? 512 * sl + 8 * lane : 0));
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool ok = has && e0 >= 0 && e0 < p.E;  // an id outside [0, E) adds nothing
    const int e = ok ? e0 : 0;

    // the rows' first loads; loads past the last row re-read it (never
    // used). Lanes past I/32 read group 0 of the row and meet a zero B operand.
    const int nrow = max(nr, 1);
    const uint8_t *pa = p.dp + (int64_t)e * p.d_sp + (on ? 16 * lane : 0);
    const uint8_t *ps = p.ds + (int64_t)e * p.d_ss + (on ? lane : 0);
    struct Row {
        u4 a;
        uint32_t s;
    };
    auto load = [&](int rr, Row &b) {
        const size_t r = (size_t)(r0 + min(rr, nrow - 1));
        b.a = ld16_stream(pa + r * IB);
        b.s = ps[r * NG];  // 48 bytes, sharing lines with the next rows' (a plain load)
    };
    Row buf[kDecDnDepth];
#pragma unroll
    for (int d = 0; d < kDecDnDepth; ++d) load(d, buf[d]);

    // the routing weights and the shared activation (4 I_s <= 64 NW
    // elements: one float4 per thread at most), loaded now and written to
    // LDS after the routed rows
    const int tk = min((int)threadIdx.x, p.K - 1);
    const int ek = p.idx[tk];
    const float wkv = p.w[tk];
    float4 ashv = float4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (NSS > 0)
        ashv = reinterpret_cast<const float4 *>(p.ash)[min((int)threadIdx.x, (p.Is >> 2) - 1)];

    // rows r .. r + 3; NEXT: issue each row's successor in the ring (the
    // last group issues none: a load past the last row would re-read a row
    // the streaming loads have not kept)
    auto four = [&](int r, auto next_c) {
        constexpr bool NEXT = decltype(next_c)::value;
        prio_left(nrow - r, nrow);
        v4f acc[kDecDnDepth];
#pragma unroll
        for (int d = 0; d < kDecDnDepth; ++d) {
            const bool drop = buf[d].s == 255u;  // E8M0 255: the group contributes nothing
            const u4 a = buf[d].a;
            const u4 av = drop ? u4{0u, 0u, 0u, 0u} : a;
            const int sa = drop ? 127 : (int)buf[d].s;
            const v8i A = v8i{(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
            acc[d] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < kDecTerms; ++t) acc[d] = mfma_fp4_fp8(A, bt[t], acc[d], sa, bs[t]);
            if constexpr (NEXT) load(r + d + kDecDnDepth, buf[d]);
        }
        const float y = diag_sum4(acc);  // lane group k: row r + k
        const int rk = r + (lane >> 4);
        if ((lane & 15) == 0 && rk < nr && has) y_l[wave * p.RB + rk] = ok ? y : 0.0f;
    };
    int r = 0;
    for (; r + kDecDnDepth < nrow; r += kDecDnDepth) four(r, std::true_type{});
    four(r, std::false_type{});
    __builtin_amdgcn_s_setprio(0);
    if (threadIdx.x < p.K) wk_l[threadIdx.x] = (ek >= 0 && ek < p.E) ? wkv : 0.0f;
    if (4 * (int)threadIdx.x < p.Is) reinterpret_cast<float4 *>(ash_l)[threadIdx.x] = ashv;
    __syncthreads();  // the staged weights and activation
    if constexpr (NSS > 0) {  // the shared rows: fp32 products in slice order, one wave-wide sum per row
#pragma unroll
        for (int k = 0; k < kDecShRows; ++k) {
            float acc = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NSS; ++sl) {
                const bool son = 512 * sl + 8 * lane < p.Is;
                const int i = son ? 512 * sl + 8 * lane : 0;
                const uint32_t msk = lane_mask(son);  // off lanes: a zero activation
                const u4 a0 = ld16m(ash_l + i, msk), a1 = ld16m(ash_l + i + 4, msk);
                const u4 w = shw[k][sl];
                acc = fmaf(bf16f(w[0] & 0xffffu), __uint_as_float(a0.x), acc);
                acc = fmaf(bf16f(w[0] >> 16), __uint_as_float(a0.y), acc);
                acc = fmaf(bf16f(w[1] & 0xffffu), __uint_as_float(a0.z), acc);
                acc = fmaf(bf16f(w[1] >> 16), __uint_as_float(a0.w), acc);
                acc = fmaf(bf16f(w[2] & 0xffffu), __uint_as_float(a1.x), acc);
                acc = fmaf(bf16f(w[2] >> 16), __uint_as_float(a1.y), acc);
                acc = fmaf(bf16f(w[3] & 0xffffu), __uint_as_float(a1.z), acc);
                acc = fmaf(bf16f(w[3] >> 16), __uint_as_float(a1.w), acc);
            }
            acc = wave_sum(acc);
            if (lane == 0) sh_l[wave + kDecDnWaves * k] = acc;
        }
    }
    __syncthreads();

    // router-order sum (ids outside [0, E) add nothing), the shared row, the epilogue
    for (int r = threadIdx.x; r < nr; r += blockDim.x) {
        float acc = 0.0f;
        for (int j = 0; j < p.K; ++j) acc = fmaf(wk_l[j], y_l[j * p.RB + r], acc);  // a dropped slot: 0 * 0
        if (NSS > 0) acc += sh_l[r];  // row r0 + r: wave r % NW, k = r / NW
        float *op = p.out + r0 + r;
        if (p.resid) acc = *op + acc;
        *op = acc;
        if (p.ob) p.ob[r0 + r] = bf16_rne(acc);
    }
    // ids outside [0, E), counted once: thread j of block 0 checks slot j
    // (the id it already holds; a serial loop of loads here would hold the
    // block's end by one cache round trip per slot)
    if (blockIdx.x == 0 && threadIdx.x < p.K && (ek < 0 || ek >= p.E)) atomicAdd(p.errors, 1ull);
}


// ---------------------------------------------------------------------------
// Gate/up of a batch's light experts that hold one or two assignments (NT):
// G's routed rows without the top-k and the shared rows. Block (item li,
// unit qb) takes rows [32 qb, 32 qb + 32) of gate and up of the item's expert
// for its NT tokens; wave w streams one matrix (w & 1) over 16 rows (w >> 1),
// two rows in flight, each 1 KB row piece as 4 bf16 MFMAs per token after the
// exact fp4 -> bf16 expansion (the diagonal dot product), the first token at
// the lanes' K positions in registers, the second read from LDS per use;
// wave 0 then writes the 32 NT activations as bf16 hi and lo, the rows the
// streamed down projection reads. The rows are read in whole 1 KB pieces
// (the many-token streaming kernel reads 64 bytes of 16 rows per
// instruction), so the streaming loads apply.
struct GuOneParams {
    const uint8_t *gp, *gs, *up, *us;
    int64_t g_sp, g_ss, u_sp, u_ss;
    int H, I, K, act;
    float b1, b2;
    const uint16_t *x;                             // tokens, bf16 [T][H]
    const int32_t *active_e, *active_off, *sorted;
    const int32_t *items, *items_n;                // the items (active-list positions), their count
    uint16_t *act_hi, *act_lo;                     // [assignment][I]
};

// the 4 waves' E8M0 rows, the sums [NT][4][16], the tokens [NT][NS][64] u4
__host__ __device__ constexpr int gu_one_lds_bytes(int H, int NS, int NT)
{
    return 2 * H + NT * 4 * 16 * 4 + NT * NS * 64 * 16;
}

// NS: 512-element token slices (H <= 512 NS); NT: assignments per item (1, 2)
template <int NS, int NT>
__global__ __launch_bounds__(256, 3) void k_gu_one(GuOneParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int NG = p.I >> 5;
    const int li = blockIdx.x / NG, qb = blockIdx.x - li * NG;
    if (li >= *p.items_n) return;  // the grid covers the most items a batch can have
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = p.H, HB = H >> 1, HG = H >> 5;  // packed bytes and E8M0 groups per row
    const int mat = wave & 1, half = wave >> 1;
    uint8_t *sc_l = lds + wave * (H / 2);                                  // this wave's 16 E8M0 rows
    float *sum_l = reinterpret_cast<float *>(lds + 2 * H);                 // [NT][4][16]
    u4 *x_l = reinterpret_cast<u4 *>(sum_l + NT * 4 * kDecUnitRows);       // [NT][NS][64]
    const int q = p.items[li];
    const int e = p.active_e[q], off = p.active_off[q];

    // the rows' first loads, the wave's 16 E8M0 rows (contiguous), the tokens
    const int row0 = 32 * qb + kDecUnitRows * half;
    const uint8_t *sbase = (mat ? p.us + (int64_t)e * p.u_ss : p.gs + (int64_t)e * p.g_ss) + (size_t)row0 * HG;
    const uint8_t *wbase = (mat ? p.up + (int64_t)e * p.u_sp : p.gp + (int64_t)e * p.g_sp) + (size_t)row0 * HB;
    int soff[kDecGuPieces];        // this lane's offset in a row piece (off lanes: the last on lane's)
    int gidx[kDecGuPieces];        // this lane's E8M0 group (off lanes: 0)
    uint32_t smask[kDecGuPieces];  // off lanes scale their weights by 0
#pragma unroll
    for (int s = 0; s < kDecGuPieces; ++s) {
        const bool on = 64 * s + lane < HG;
        soff[s] = min(1024 * s + 16 * lane, HB - 16);
        gidx[s] = on ? 64 * s + lane : 0;
        smask[s] = lane_mask(on);
    }
    struct Row {
        u4 a[kDecGuPieces];
    };
    auto load = [&](int r, Row &b) {
        const size_t ro = (size_t)r * HB;
#pragma unroll
        for (int s = 0; s < kDecGuPieces; ++s) b.a[s] = ld16_stream(wbase + ro + soff[s]);
    };
    // issue order: the tokens (cache hits), the E8M0 rows, then the routed
    // rows, so the LDS stores wait only for the first two and the rows stay
    // in flight across the barrier (memory counters retire in issue order)
    constexpr int XQ = (NS * 64 + 255) / 256;
    u4 xs[NT][XQ];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const uint16_t *xt = p.x + (size_t)(p.sorted[off + c] / p.K) * H;  // assignment c's token
#pragma unroll
        for (int k = 0; k < XQ; ++k) {
            const int i = threadIdx.x + 256 * k;
            const bool on = i < NS * 64 && 8 * i < H;
            xs[c][k] = ld16m(xt + (on ? 8 * i : 0), lane_mask(on));
        }
    }
    constexpr int SQ = 8192 / 2 / 1024;  // 16-byte pieces per lane (H <= 8192)
    u4 scv[SQ];
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        const int i = 16 * lane + 1024 * k;
        scv[k] = ld16_stream(sbase + min(i, H / 2 - 16));  // off lanes: the last on lane's address
    }
    __builtin_amdgcn_sched_barrier(0);  // keeps that issue order
    constexpr int GD = 2;  // rows in flight
    Row bq[GD];
#pragma unroll
    for (int d = 0; d < GD; ++d) load(d, bq[d]);
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int k = 0; k < XQ; ++k) {
            const int i = threadIdx.x + 256 * k;
            if (i < NS * 64) x_l[c * NS * 64 + i] = xs[c][k];
        }
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        const int i = 16 * lane + 1024 * k;
        if (i < H / 2) *reinterpret_cast<u4 *>(sc_l + i) = scv[k];
    }
    __syncthreads();  // the token slices and this wave's E8M0 rows

    // the first token at this lane's K positions (lane l of row piece s:
    // elements 2048 s + 32 l + [0, 32)); an off lane's weights are scaled by
    // 0, so what it reads for a token does not matter (index 0)
    u4 xv[kDecGuPieces][4];
#pragma unroll
    for (int s = 0; s < kDecGuPieces; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = 2048 * s + 32 * lane + 8 * c;
            xv[s][c] = ld16m(x_l + (i < H ? i / 8 : 0), lane_mask(i < H));
        }

    float mine[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) mine[c] = 0.0f;
    auto compute = [&](int r, const Row &b) {
        v4f acc[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // the second token's slice base, opaque to the compiler: its reads
        // are the same for every row and would otherwise be hoisted out of
        // the unrolled row loop into 64 registers (it spilled)
        int x1 = NS * 64;
        asm volatile("" : "+v"(x1));
#pragma unroll
        for (int s = 0; s < kDecGuPieces; ++s) {
            const float f = __uint_as_float(__float_as_uint(e8m0_to_f32(sc_l[r * HG + gidx[s]])) & smask[s]);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf8 a = dequant8_bf16(b.a[s][st], f);
                acc[0] = mfma_bf16(a, as_bf8(xv[s][st]), acc[0]);
                if constexpr (NT > 1) {
                    const int i = 2048 * s + 32 * lane + 8 * st;
                    acc[1] = mfma_bf16(a, as_bf8(x_l[x1 + (i < H ? i / 8 : 0)]), acc[1]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const float v = diag_sum(acc[c]);
            mine[c] = lane == r ? v : mine[c];
        }
    };
    // fully unrolled: the rows' next loads stop at the last row
#pragma unroll
    for (int r = 0; r < kDecUnitRows; r += GD) {
        prio_left(kDecUnitRows - r, kDecUnitRows);
#pragma unroll
        for (int d = 0; d < GD; ++d) {
            compute(r + d, bq[d]);
            if (r + d + GD < kDecUnitRows) load(r + d + GD, bq[d]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (lane < kDecUnitRows)
#pragma unroll
        for (int c = 0; c < NT; ++c) sum_l[(c * 4 + wave) * kDecUnitRows + lane] = mine[c];
    __syncthreads();

    // wave 0, lane l < 32 NT: assignment c = l / 32, row 32 qb + l % 32
    // (half (l % 32) / 16, row l % 16)
    if (wave == 0 && lane < 32 * NT) {
        const int c = lane >> 5, ll = lane & 31, hl = ll >> 4, rl = ll & 15;
        const float g = sum_l[(c * 4 + 2 * hl) * kDecUnitRows + rl];
        const float u = sum_l[(c * 4 + 2 * hl + 1) * kDecUnitRows + rl];
        const float a = act_fn(g, u, p.act, p.b1, p.b2);
        const uint16_t h = bf16_rne(a);
        const size_t o = (size_t)(off + c) * p.I + 32 * qb + ll;
        p.act_hi[o] = h;
        p.act_lo[o] = bf16_rne(a - bf16f(h));
    }
}

}  // namespace

// The shapes the three kernels take: a flat layer, H <= 8192 (four 1 KB
// pieces per gate/up row, sixteen 512-element router slices), I <= 2048 (a
// down row in one wave instruction), I_s <= 2048, top-k <= 16 (one slot per
// down wave).
bool decode_fused_ok(const LayerView &L)
{
    return L.Lt == 0 && L.H <= 8192 && L.H % 128 == 0 && L.I <= 2048 && L.I % 128 == 0 && L.Is <= 2048 &&
           L.K <= kDecDnWaves && L.E <= kMaxExperts && 32 * L.H >= L.I &&
           L.Is <= kDecShPairs * L.K * (L.I / 32);  // a block's share of the shared rows fits its LDS
}

// Workspace use (the T = 1 layout): sc, ch; ash; the e4m3 terms in act
// (k * 4 * I bytes); their E8M0 scales in ys.
hipError_t launch_decode_fused(const LayerView &L, const uint16_t *x, int32_t *idx, float *w, float *logits,
                               bool route, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                               Profiler *prof, const OutEpi &epi, bool routed)
{
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    float *sc = reinterpret_cast<float *>(ws + lay.sc);
    float *ch = reinterpret_cast<float *>(ws + lay.ch);
    float *ash = reinterpret_cast<float *>(ws + lay.ash);
    uint8_t *aq = reinterpret_cast<uint8_t *>(ws + lay.act);
    uint8_t *as = reinterpret_cast<uint8_t *>(ws + lay.ys);

    // R: the router rows (logits, scores)
    if (route && !routed) {
        StageMark m(prof, K3MOE_STAGE_ROUTER, s);
        if (launch_router_t1(L, x, sc, ch, logits, s) != hipSuccess) return hipGetLastError();
    }
    // the top-k in G (16 experts per lane, 16-byte loads) or on its own
    const bool fused_topk = route && L.E > 512 && L.E <= 1024 && L.E % 4 == 0;
    if (route && !fused_topk) {
        StageMark m(prof, K3MOE_STAGE_TOPK, s);
        if (launch_topk(L, 1, sc, ch, idx, w, s) != hipSuccess) return hipGetLastError();
    }
    // G: top-k, routed gate/up
    {
        StageMark m(prof, K3MOE_STAGE_GATEUP, s);
        DecGuParams gp{};
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
        gp.E = L.E;
        gp.K = L.K;
        gp.act = L.act;
        gp.b1 = L.b1;
        gp.b2 = L.b2;
        gp.renorm = L.renorm;
        gp.rscale = L.routed_scale;
        gp.x = x;
        gp.sc = sc;
        gp.ch = ch;
        gp.idx = idx;
        gp.w = w;
        gp.aq = aq;
        gp.as = as;
        gp.sh_gate = L.sh_gate;
        gp.sh_up = L.sh_up;
        gp.ash = ash;
        gp.Is = L.Is;
        const unsigned nb = (unsigned)(L.K * (L.I / 32));
        const int NS = L.H <= 2048 ? 4 : L.H <= 4096 ? 8 : L.H <= 7168 ? 14 : 16;
        const size_t lds = dec_gu_lds_bytes(L.H, NS);
#define K3_GU(NQ, NSL) k_dec_gateup<NQ, NSL><<<nb, 256, lds, s>>>(gp)
        if (fused_topk) {
            if (NS == 4) K3_GU(16, 4); else if (NS == 8) K3_GU(16, 8); else if (NS == 14) K3_GU(16, 14); else K3_GU(16, 16);
        } else {
            if (NS == 4) K3_GU(0, 4); else if (NS == 8) K3_GU(0, 8); else if (NS == 14) K3_GU(0, 14); else K3_GU(0, 16);
        }
#undef K3_GU
    }
    // D: shared down, routed down, router-order sum, epilogue
    {
        StageMark m(prof, K3MOE_STAGE_DOWN, s);
        DecDnParams dp{};
        dp.dp = L.dp;
        dp.ds = L.ds;
        dp.d_sp = L.d_sp;
        dp.d_ss = L.d_ss;
        dp.H = L.H;
        dp.I = L.I;
        dp.E = L.E;
        dp.K = L.K;
        // one block per CU, at most kDecShRows rows per wave
        const int nb = std::max(std::min(ncu, L.H), (L.H + kDecDnRowsMax - 1) / kDecDnRowsMax);
        dp.RB = (L.H + nb - 1) / nb;
        dp.idx = idx;
        dp.w = w;
        dp.aq = aq;
        dp.as = as;
        dp.sh_down = L.sh_down;
        dp.ash = ash;
        dp.Is = L.Is;
        dp.out = out;
        dp.resid = epi.resid;
        dp.ob = epi.ob;
        dp.errors = L.errors;
        const unsigned grid = (unsigned)((L.H + dp.RB - 1) / dp.RB);
        const size_t lds = sizeof(float) * (((L.K * dp.RB + 3) & ~3) + L.Is);
        const int nss = (L.Is + 511) / 512;
        if (nss == 0) k_dec_down<0><<<grid, 64 * kDecDnWaves, lds, s>>>(dp);
        else if (nss == 1) k_dec_down<1><<<grid, 64 * kDecDnWaves, lds, s>>>(dp);
        else if (nss == 2) k_dec_down<2><<<grid, 64 * kDecDnWaves, lds, s>>>(dp);
        else if (nss == 3) k_dec_down<3><<<grid, 64 * kDecDnWaves, lds, s>>>(dp);
        else k_dec_down<4><<<grid, 64 * kDecDnWaves, lds, s>>>(dp);
    }
    return hipGetLastError();
}


// Gate/up of the light items with nt (1 or 2) assignments (a flat layer:
// the routed input is x itself).
bool gu_one_ok(const LayerView &L) { return L.Lt == 0 && L.H <= 8192 && L.H % 128 == 0 && L.I % 32 == 0; }

hipError_t launch_gu_one(const LayerView &L, const uint16_t *x, int T, int nt, const int32_t *active_e,
                         const int32_t *active_off, const int32_t *sorted, const int32_t *items,
                         const int32_t *items_n, uint16_t *act_hi, uint16_t *act_lo, hipStream_t s)
{
    GuOneParams p{};
    p.gp = L.gp;
    p.gs = L.gs;
    p.up = L.up;
    p.us = L.us;
    p.g_sp = L.g_sp;
    p.g_ss = L.g_ss;
    p.u_sp = L.u_sp;
    p.u_ss = L.u_ss;
    p.H = L.H;
    p.I = L.I;
    p.K = L.K;
    p.act = L.act;
    p.b1 = L.b1;
    p.b2 = L.b2;
    p.x = x;
    p.active_e = active_e;
    p.active_off = active_off;
    p.sorted = sorted;
    p.items = items;
    p.items_n = items_n;
    p.act_hi = act_hi;
    p.act_lo = act_lo;
    const int64_t cap = std::min<int64_t>(L.E, (int64_t)T * L.K);  // the most items a batch can have
    const unsigned nb = (unsigned)(cap * (L.I / 32));
    const int NS = L.H <= 2048 ? 4 : L.H <= 4096 ? 8 : L.H <= 7168 ? 14 : 16;
    const size_t lds = gu_one_lds_bytes(L.H, NS, nt);
#define K3_ONE(NSL)                                                    \
    do {                                                               \
        if (nt == 1) k_gu_one<NSL, 1><<<nb, 256, lds, s>>>(p);         \
        else k_gu_one<NSL, 2><<<nb, 256, lds, s>>>(p);                 \
    } while (0)
    if (NS == 4) K3_ONE(4);
    else if (NS == 8) K3_ONE(8);
    else if (NS == 14) K3_ONE(14);
    else K3_ONE(16);
#undef K3_ONE
    return hipGetLastError();
}

}  // namespace k3moe
