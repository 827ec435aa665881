// Device helpers shared by the gfx950 kernel files: vector types, bf16 and
// E8M0 conversions, the fp4 -> bf16 expansion, MFMA wrappers and the
// operands of the scaled MFMA, the e4m3 term expansion, the gated
// activation, wave-level reductions and the top-k of one token.
#pragma once

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "k3moe.h"

namespace k3moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// Loads of weights that one call reads once, marked nontemporal: the caches
// treat them as streaming, so they neither evict what the caches hold for
// the rest of the call nor cost allocation in the last-level cache (8-layer
// decode stack: 0.597 -> 0.560 ms per step). Only for loads whose wave
// instruction covers whole 128-byte lines: a line that two instructions
// share (the streaming GEMV kernels read 64 bytes of a row per
// instruction) is gone before the second one asks for it (those kernels ran
// 25-30 % slower with the hint).
__device__ __forceinline__ u4 ld16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p));
}

// bf16 bit pattern (low 16 bits of h) -> fp32, exactly.
__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne_u32(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return (uint16_t)bf16_rne_u32(f); }

// E8M0 byte -> the fp32 factor 2^(s-127) for the scaled converters; byte 0 is
// the subnormal 2^-127, byte 255 drops its group (factor 0).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return s == 255u ? 0.0f : __uint_as_float(s == 0u ? 0x00400000u : s << 23);
}

// 8 fp4 weights (one 32-bit word, low nibble first) -> 8 bf16, scaled
// exactly (every fp4 value times a power of two is a bf16).
__device__ __forceinline__ bf8 dequant8_bf16(uint32_t w, float scale)
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

// Scaled MFMA, A in fp4 (format 4), B in fp8 e4m3 (format 0); the scale
// bytes are taken from byte S of the packed scale words.
template <int S = 0>
__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i &a, const v8i &b, v4f c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, S, sa, S, sb);
}

// A lane's scale bytes for 4 consecutive K steps: from the 16 bytes holding
// K-blocks 4s+g (step s, lane group g) of a row, byte g of each dword.
__device__ __forceinline__ uint32_t gather_scales(u4 v, uint32_t grp)
{
    const uint32_t lo = __builtin_amdgcn_perm(v.y, v.x, grp | ((4u + grp) << 8) | 0x0c0c0000u);
    const uint32_t hi = __builtin_amdgcn_perm(v.w, v.z, 0x00000c0cu | (grp << 16) | ((4u + grp) << 24));
    return lo | hi;
}

// 0x80 in each byte of x that is 0xFF (E8M0 255), 0 elsewhere.
__device__ __forceinline__ uint32_t ff_bytes(uint32_t x)
{
    const uint32_t y = ~x;
    return ~(((y & 0x7f7f7f7fu) + 0x7f7f7f7fu) | y | 0x7f7f7f7fu);
}

// Operands of the scaled MFMA: fp4 A (16 bytes in the low 4 registers) and
// fp8 B (two 16-byte halves).
__device__ __forceinline__ v8i a_operand(u4 v) { return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

__device__ __forceinline__ v8i b_operand(u4 lo, u4 hi)
{
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Maximum over the 8 lanes of each aligned lane octet (DPP: swap neighbours,
// swap pairs, mirror the half-row).
__device__ __forceinline__ float octet_max(float m)
{
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xb1, 0xf, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4e, 0xf, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xf, 0xf, false)));
    return m;
}

// Split values into NT e4m3 terms, x = sum_t 2^(S_t - 127) q_t, in the
// layout of the scaled MFMA's fp8 operand. This lane holds NV consecutive
// values of a 32-element block whose other values sit in the lanes that
// block_max reduces over; the block shares one E8M0 scale per term. The
// scale puts the block's largest remainder in [224, 448]; a term takes only
// the elements within 6 binades of that maximum (the rest stay in the
// remainder) and each term's rounding error is carried exactly into the
// next term. code[t][q] packs the codes of values 4q..4q+3 of term t, first
// value lowest; sbyte[t] is the term's E8M0 byte.
template <int NT, int NV, class MaxFn>
__device__ __forceinline__ void split_e4m3_terms(float (&r)[NV], MaxFn block_max, uint32_t (&code)[NT][NV / 4],
                                                 int (&sbyte)[NT])
{
    static_assert(NV % 4 == 0, "whole code words");
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float lm = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) lm = fmaxf(lm, fabsf(r[i]));
        const float m = block_max(lm);
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
#pragma unroll
        for (int w = 0; w < NV / 4; ++w) {
            uint32_t c4 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float q = ldexpf(r[4 * w + i], -S);
                if (fabsf(q) >= keep_min) {
                    const uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xffu;
                    r[4 * w + i] -= ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)c, 0), S);
                    c4 |= c << (8 * i);
                }
            }
            code[t][w] = c4;
        }
        sbyte[t] = S + 127;
    }
}

// The octet form: the 8 lanes of an aligned lane octet hold one 32-element
// block, 4 consecutive values each.
template <int NT>
__device__ __forceinline__ void split_e4m3_octet(const float4 v, uint32_t (&code4)[NT], int (&sbyte)[NT])
{
    float r[4] = {v.x, v.y, v.z, v.w};
    uint32_t code[NT][1];
    split_e4m3_terms<NT, 4>(r, [](float m) { return octet_max(m); }, code, sbyte);
#pragma unroll
    for (int t = 0; t < NT; ++t) code4[t] = code[t][0];
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Gated activation (README §9, k3_situ_glu): SiTU-GLU (the sigmoid on the
// raw gate) or SwiGLU, fp32.
__device__ __forceinline__ float act_fn(float g, float u, int kind, float b1, float b2)
{
    const float sg = 1.0f / (1.0f + expf(-g));
    if (kind == K3MOE_ACT_SITU) return (b1 * tanhf(g / b1) * sg) * (b2 * tanhf(u / b2));
    return g * sg * u;
}

// Wave priority from the work this wave has left (0..3): waves that share a
// SIMD are issued oldest first at equal priority, so without this the oldest
// finishes first and the youngest runs its last rows with nobody to hide
// its loads behind.
__device__ __forceinline__ void prio_left(int left, int total)
{
    const int lv = (4 * left - 1) / total;  // left in (0, total]: 3 .. 0
    if (lv >= 3) __builtin_amdgcn_s_setprio(3);
    else if (lv == 2) __builtin_amdgcn_s_setprio(2);
    else if (lv == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// Orders LDS traffic of one wave: its earlier LDS stores are complete and
// visible to every lane of the wave before its later LDS loads (the wave's
// LDS operations complete in order; the clobber stops the compiler moving
// memory operations across).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wave-wide max / min of a uint32 through DPP (row-local steps, then the
// row broadcasts), read back from lane 63: the same value in every lane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v)
{
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast15
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving uint32 key of a selection score (> 0 for every float;
// NaN ranks as -inf).
__device__ __forceinline__ uint32_t order_key(float v)
{
    if (v != v) v = -INFINITY;
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS a wave's top-k works in.
struct TopkLds {
    uint64_t cc[64];   // candidates: key << 32 | ~expert
    float cs[64];      // their unbiased scores
    int pi[64];        // picks in router order: expert, score
    float ps[64];
};

// Top-k of one token (README §9, k3_router): the k largest selection scores
// ch, in descending order, equal scores by ascending expert index (the order
// of a repeated strict maximum); weights are the unbiased scores sc of the
// picks, renormalised in router order when renorm is set, then scaled.
// One wave; lane l holds the scores of experts l*NQ .. l*NQ+NQ-1 (a
// contiguous range, so a lower lane always holds lower expert indices) as
// order-preserving keys.
//
// Threshold and rank: tau = the k-th largest of the 64 lane maxima (a
// bitwise search on ballots). k lanes hold a key >= tau, so the k-th largest
// key is >= tau and every pick is among the candidates {key >= tau}. When
// there are at most 64 candidates (the usual case: about k of them), they
// are gathered one per lane through LDS, each takes its rank in the order
// above by comparing against every candidate (broadcast by readlane), and
// the first k ranks are the picks. A candidate is one 64-bit word, key in the
// high half and the complement of its expert index in the low half, so that
// order is a single unsigned comparison. With more candidates (heavy ties)
// the wave falls back to k rounds of a wave-wide maximum, the lowest lane
// holding it winning and rescanning its keys.
//
// topk_load issues the loads of a lane's selection scores (raw) and scores
// (sv); topk_rank then takes the top-k from them, so a kernel can put other
// work between the two. Returns, in lane j < k, pick j's expert (*pick) and
// weight (*wt). V4: E a multiple of 4 and rows 16-byte aligned (16-byte loads).
template <int NQ, bool V4>
__device__ __forceinline__ void topk_load(const float *__restrict__ sc, const float *__restrict__ ch, int E,
                                          float (&raw)[NQ], float (&sv)[NQ])
{
    const int lane = threadIdx.x & 63;
    const int e0 = lane * NQ;
    // the selection scores and the scores are loaded together, every load
    // issued before the first is used (clamped index, no branch)
    if constexpr (V4) {
#pragma unroll
        for (int q = 0; q < NQ; q += 4) {
            const int b = min(e0 + q, E - 4);
            const float4 a = *reinterpret_cast<const float4 *>(ch + b);
            const float4 d = *reinterpret_cast<const float4 *>(sc + b);
            raw[q] = a.x, raw[q + 1] = a.y, raw[q + 2] = a.z, raw[q + 3] = a.w;
            sv[q] = d.x, sv[q + 1] = d.y, sv[q + 2] = d.z, sv[q + 3] = d.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            raw[q] = ch[min(e0 + q, E - 1)];
            sv[q] = sc[min(e0 + q, E - 1)];
        }
    }
}

template <int NQ>
__device__ __forceinline__ void topk_rank(const float (&raw)[NQ], const float (&sv)[NQ], int E, int K, int renorm,
                                          float rscale, TopkLds &L, int *pick, float *wt)
{
    const int lane = threadIdx.x & 63;
    const int e0 = lane * NQ;
    uint32_t v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = e0 + q < E ? order_key(raw[q]) : 0u;  // 0: none / taken
    uint32_t lm = 0u;
#pragma unroll
    for (int q = 0; q < NQ; ++q) lm = v[q] > lm ? v[q] : lm;

    // tau: the k-th largest of the 64 lane maxima, i.e. the largest t with
    // at least k lane maxima >= t, found bit by bit on the wave's ballots (no
    // memory round trip)
    uint32_t tau = 0u;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = tau | (1u << b);
        if (__popcll(__ballot(lm >= c)) >= K) tau = c;
    }

    // gather the candidates (key >= tau; a key of 0 is no expert): candidate
    // i goes to slot i of the LDS list
    int C = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const bool in = v[q] >= tau && v[q] != 0u;
        const uint64_t m = __ballot(in);
        const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (in && pos < 64) {
            L.cc[pos] = ((uint64_t)v[q] << 32) | (uint32_t)~(uint32_t)(e0 + q);
            L.cs[pos] = sv[q];
        }
        C += __popcll(m);
    }
    wave_lds_sync();

    int mine = 0;
    float mine_s = 0.0f;  // score of pick j, held by lane j
    if (C <= 64) {
        // lane i holds candidate i; its rank is the number of larger
        // candidates, counted against each candidate broadcast in turn
        const uint64_t k0 = lane < C ? L.cc[lane] : 0ull;
        const float s0 = lane < C ? L.cs[lane] : 0.0f;
        const uint32_t k0h = (uint32_t)(k0 >> 32), k0l = (uint32_t)k0;
        int r = 0;
        for (int j = 0; j < C; ++j) {
            const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)k0h, j) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)k0l, j);
            r += kj > k0 ? 1 : 0;
        }
        if (lane < C && r < K) {
            L.pi[r] = (int)~(uint32_t)k0;
            L.ps[r] = s0;
        }
        wave_lds_sync();
        if (lane < K) {
            mine = L.pi[lane];
            mine_s = L.ps[lane];
        }
    } else {
        uint32_t bk;  // best remaining key of this lane (0: none)
        int bq;       // its position
        auto rescan = [&]() {
            bk = 0u;
            bq = 0;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const bool gt = v[q] > bk;
                bk = gt ? v[q] : bk;
                bq = gt ? q : bq;
            }
        };
        rescan();
        for (int j = 0; j < K; ++j) {
            const uint32_t m = wave_reduce_u32<true>(bk);
            const uint64_t holders = __ballot(bk == m);
            const int wl = (int)__builtin_ctzll(holders);  // lowest lane holding the maximum
            const int win = wl * NQ + __builtin_amdgcn_readlane(bq, wl);
            float ws = 0.0f;
            if (lane == wl) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if (q == bq) {
                        ws = sv[q];
                        v[q] = 0u;
                    }
                rescan();
            }
            ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws), wl));
            if (lane == j) {
                mine = win;
                mine_s = ws;
            }
        }
    }
    // renormalisation: the sum runs over the picks in router order
    float s = 0.0f;
    for (int j = 0; j < K; ++j) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine_s), j));
    float v0 = mine_s;
    if (renorm && s > 0.0f) v0 /= s;
    *pick = mine;
    *wt = v0 * rscale;
}

template <int NQ, bool V4>
__device__ __forceinline__ void topk_wave(const float *__restrict__ sc, const float *__restrict__ ch, int E, int K,
                                          int renorm, float rscale, TopkLds &L, int *pick, float *wt)
{
    float raw[NQ], sv[NQ];
    topk_load<NQ, V4>(sc, ch, E, raw, sv);
    topk_rank<NQ>(raw, sv, E, K, renorm, rscale, L, pick, wt);
}

// Router epilogue for one (token, expert): the fp32 logit, the fp32 score
// (sigmoid evaluated in fp64, rounded once) and the fp32 selection score.
__device__ __forceinline__ void router_finish(double acc, int t, int e, int E, const float *__restrict__ bias,
                                              float *__restrict__ sc, float *__restrict__ ch,
                                              float *__restrict__ logits)
{
    const float l32 = (float)acc;
    const float s = (float)(1.0 / (1.0 + exp(-(double)l32)));
    const size_t o = (size_t)t * E + e;
    sc[o] = s;
    ch[o] = s + (bias ? bias[e] : 0.0f);
    if (logits) logits[o] = l32;
}

}  // namespace k3moe
