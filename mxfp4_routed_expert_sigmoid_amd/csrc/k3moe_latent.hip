// The latent layer's own steps (the "kimi-k3-in-c" README, §9 "Picking 16
// experts of 896", k3_moe steps 2, 4 and 5; §5 "Kernels with a floating point
// contract", k3_rmsnorm): the bf16 down-projection of x into the experts'
// latent, the RMSNorm of the routed aggregate, the bf16 up-projection back to
// the hidden width. The routing, the experts, the shared expert and the
// router-order sum are the flat layer's kernels.
#include <algorithm>

#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {


// ---------------------------------------------------------------------------
// Projection with bf16 weights W [R][Kd] of NP token planes [T][Kd] (bf16; two
// planes carry the hi and lo of an fp32 input and go into one accumulator):
// part[s][t][r] = sum over K slice s of W[r][k] * (sum of the planes)[t][k].
// Block: 4 waves x 16 rows, 64 tokens, one K slice (grid z) walked in chunks
// of 128; each lane's weight fragment comes from HBM into registers once per
// chunk (one chunk ahead), the tokens through double-buffered LDS. Slices
// give small batches enough blocks to stream the weights at full width; their
// fp32 sums are added in slice order by k_proj_finish.
//
// K mapping: lane group g (lanes 16g..16g+15) holds K = 128c + 32st + 8g +
// [0, 8) of MFMA step st of chunk c on both sides (v_mfma_f32_16x16x32_bf16:
// lane l holds A row l % 16 and B column l % 16).
constexpr int kPjRows = 64;    // rows per block (4 waves x 16)
constexpr int kPjTok = 64;     // tokens per block
constexpr int kPjKC = 128;     // K per chunk
constexpr int kPjPad = 16;     // LDS bytes after each token row
constexpr int kPjRow = kPjKC * 2 + kPjPad;

__host__ __device__ constexpr int proj_lds_bytes(int np) { return 2 * np * kPjTok * kPjRow; }

template <int NP>
__global__ __launch_bounds__(256) void k_proj(const uint16_t *__restrict__ W, const uint16_t *__restrict__ p0,
                                              const uint16_t *__restrict__ p1, int T, int R, int Kd, int kspan,
                                              float *__restrict__ part)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int r0 = blockIdx.x * kPjRows + wave * 16, t0 = blockIdx.y * kPjTok;
    const int k0 = blockIdx.z * kspan, k1 = min(Kd, k0 + kspan);
    const int NCH = (k1 - k0) / kPjKC;
    const uint8_t *wrow = reinterpret_cast<const uint8_t *>(W) + ((size_t)min(r0 + l16, R - 1) * Kd + k0) * 2 + 16 * g;
    const uint8_t *pp[2] = {reinterpret_cast<const uint8_t *>(p0), reinterpret_cast<const uint8_t *>(p1)};

    // token staging: thread -> (plane, token, 16-byte segment) of a chunk
    constexpr int SEG = kPjKC * 2 / 16;                         // 16 per token row
    constexpr int NB = NP * kPjTok * SEG / 256;                 // u4 per thread
    u4 xs[NB];
    auto bload = [&](int c) {
        const int cc = min(c, NCH - 1);
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + 256 * q;
            const int pl = v / (kPjTok * SEG), vv = v - pl * (kPjTok * SEG);
            const int col = vv / SEG, seg = vv - col * SEG;
            const int t = min(t0 + col, T - 1);
            xs[q] = *reinterpret_cast<const u4 *>(pp[pl] + ((size_t)t * Kd + k0 + cc * kPjKC) * 2 + 16 * seg);
        }
    };
    auto bstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v = tid + 256 * q;
            const int pl = v / (kPjTok * SEG), vv = v - pl * (kPjTok * SEG);
            const int col = vv / SEG, seg = vv - col * SEG;
            *reinterpret_cast<u4 *>(lds + ((buf * NP + pl) * kPjTok + col) * kPjRow + 16 * seg) = xs[q];
        }
    };
    struct Chunk {
        u4 a[4];
    };
    auto aload = [&](int c, Chunk &b) {
        const int cc = min(c, NCH - 1);
#pragma unroll
        for (int st = 0; st < 4; ++st) b.a[st] = *reinterpret_cast<const u4 *>(wrow + (cc * kPjKC + 32 * st) * 2);
    };
    v4f acc[4];
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) acc[tf] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const Chunk &b, int buf) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf8 a = as_bf8(b.a[st]);
#pragma unroll
            for (int tf = 0; tf < 4; ++tf)
#pragma unroll
                for (int pl = 0; pl < NP; ++pl) {
                    const bf8 bv = as_bf8(*reinterpret_cast<const u4 *>(
                        lds + ((buf * NP + pl) * kPjTok + 16 * tf + l16) * kPjRow + (32 * st + 8 * g) * 2));
                    acc[tf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[tf], 0, 0, 0);
                }
        }
    };

    if (NCH > 0) {
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
    }
    // lane holds rows 4g + i of token column 16 tf + l16
    if (r0 >= R) return;
    float *ps = part + (size_t)blockIdx.z * T * R;
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
        const int t = t0 + 16 * tf + l16;
        if (t < T)
            *reinterpret_cast<float4 *>(ps + (size_t)t * R + r0 + 4 * g) =
                float4{acc[tf][0], acc[tf][1], acc[tf][2], acc[tf][3]};
    }
}

// Slices added in order, then the addend's AS slices in order: fp32 out
// [T][R], or bf16 hi/lo planes.
__global__ __launch_bounds__(256) void k_proj_finish(const float *__restrict__ part, int S, int T, int R,
                                                     const float *__restrict__ addend, int AS, float *__restrict__ out,
                                                     uint16_t *__restrict__ hi, uint16_t *__restrict__ lo, int resid,
                                                     uint16_t *__restrict__ ob)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x, n = (int64_t)T * R;
    if (i >= n) return;
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(size_t)s * n + i];
    if (addend) {
        float a = addend[i];
        for (int s = 1; s < AS; ++s) a += addend[(size_t)s * n + i];
        v += a;
    }
    if (out) {
        if (resid) v = out[i] + v;  // the residual stream: h + (complete layer output)
        out[i] = v;
        if (ob) ob[i] = bf16_rne(v);
    } else {
        const uint16_t h = bf16_rne(v);
        hi[i] = h;
        lo[i] = bf16_rne(v - bf16f(h));
    }
}

// RMSNorm of the routed aggregate (k3_rmsnorm: sum of squares in fp64,
// epsilon inside the root, x * inv * gamma in fp32), then bf16 hi and lo
// planes for the up-projection. One block per token; L % 4 == 0. Each pass
// issues its loads kRmsV float4 per thread at a time, so a pass over a row of
// up to 4096 costs one memory latency.
constexpr int kRmsV = 4;
template <bool NORM>
__global__ __launch_bounds__(256) void k_rms_split(const float *__restrict__ acc, int L, const float *__restrict__ gamma,
                                                   float eps, uint16_t *__restrict__ hi, uint16_t *__restrict__ lo)
{
    __shared__ double red[4];
    __shared__ float inv_sh;
    const int t = blockIdx.x, tid = threadIdx.x, nv = L / 4;
    const float4 *a = reinterpret_cast<const float4 *>(acc + (size_t)t * L);
    float inv = 1.0f;
    if constexpr (NORM) {
        double ss = 0.0;
        for (int c0 = 0; c0 < nv; c0 += 256 * kRmsV) {
            float4 v[kRmsV];
#pragma unroll
            for (int j = 0; j < kRmsV; ++j) {
                const int i = c0 + tid + 256 * j;
                v[j] = i < nv ? a[i] : float4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int j = 0; j < kRmsV; ++j) {
                ss = fma((double)v[j].x, (double)v[j].x, ss);
                ss = fma((double)v[j].y, (double)v[j].y, ss);
                ss = fma((double)v[j].z, (double)v[j].z, ss);
                ss = fma((double)v[j].w, (double)v[j].w, ss);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        if (tid == 0) inv_sh = (float)(1.0 / sqrt((red[0] + red[1] + red[2] + red[3]) / (double)L + (double)eps));
        __syncthreads();
        inv = inv_sh;
    }
    const float4 *gm = reinterpret_cast<const float4 *>(gamma);
    uint2 *h2 = reinterpret_cast<uint2 *>(hi + (size_t)t * L), *l2 = reinterpret_cast<uint2 *>(lo + (size_t)t * L);
    for (int c0 = 0; c0 < nv; c0 += 256 * kRmsV) {
        float4 v[kRmsV], gv[kRmsV];
#pragma unroll
        for (int j = 0; j < kRmsV; ++j) {
            const int i = min(c0 + tid + 256 * j, nv - 1);
            v[j] = a[i];
            if constexpr (NORM) gv[j] = gm[i];
        }
#pragma unroll
        for (int j = 0; j < kRmsV; ++j) {
            const int i = c0 + tid + 256 * j;
            if (i >= nv) break;
            float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            if constexpr (NORM) {
                f[0] = f[0] * inv * gv[j].x;
                f[1] = f[1] * inv * gv[j].y;
                f[2] = f[2] * inv * gv[j].z;
                f[3] = f[3] * inv * gv[j].w;
            }
            uint16_t h[4], l[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                h[q] = bf16_rne(f[q]);
                l[q] = bf16_rne(f[q] - bf16f(h[q]));
            }
            h2[i] = uint2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
            l2[i] = uint2{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16)};
        }
    }
}

// ---------------------------------------------------------------------------
// One token: both projections as streaming matrix-vector products with fp32
// FMA (a one-column product leaves the MFMA nothing to gain). A wave owns RW
// consecutive weight rows over the whole K range, walked in slices of 512
// (16 bytes = 8 weights of each row per lane), kGvDepth slices in flight;
// the per-lane sums are reduced across the wave at the end. The token side
// (the bf16 x, or the normed fp32 aggregate) is read per slice and stays in
// the caches.
constexpr int kGvWaves = 4;
constexpr int kGvDepth = 4;    // slices in flight per wave
constexpr int kGvSlice = 512;  // K per slice (64 lanes x 8)

__device__ __forceinline__ float gv_wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Rows row0 .. row0 + RW - 1 (clamped to R) of W [R][K] times the token:
// NORMED = false: bf16 x [K]; NORMED = true: fp32 a[k] * inv * gamma[k]
// (gamma null: a[k] * inv). inv is computed by the block (fp64 sum of
// squares, epsilon inside the root) after the first weight slices are in
// flight, when want_norm is set; every block computes the same value.
template <int RW, bool NORMED>
__device__ __forceinline__ void gv_rows(const uint16_t *__restrict__ W, int R, int K, int row0,
                                        const uint16_t *__restrict__ x, const float *__restrict__ a,
                                        const float *__restrict__ gamma, bool want_norm, float eps,
                                        float (&acc)[RW])
{
    __shared__ double red[kGvWaves];
    __shared__ float inv_sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int NS = (K + kGvSlice - 1) / kGvSlice;
    const uint16_t *wr[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        wr[q] = W + (size_t)min(row0 + q, R - 1) * K;
        acc[q] = 0.0f;
    }
    u4 buf[kGvDepth][RW];
    auto load = [&](int sl, u4(&b)[RW]) {
        const int i = min(sl * kGvSlice + lane * 8, K - 8);
#pragma unroll
        for (int q = 0; q < RW; ++q) b[q] = *reinterpret_cast<const u4 *>(wr[q] + i);
    };
#pragma unroll
    for (int d = 0; d < kGvDepth; ++d) load(min(d, NS - 1), buf[d]);

    float inv = 1.0f;
    if constexpr (NORMED) {
        if (want_norm) {
            double ss = 0.0;
            for (int l4 = tid; l4 < K / 4; l4 += 64 * kGvWaves) {
                const float4 v = reinterpret_cast<const float4 *>(a)[l4];
                ss = fma((double)v.x, (double)v.x, ss);
                ss = fma((double)v.y, (double)v.y, ss);
                ss = fma((double)v.z, (double)v.z, ss);
                ss = fma((double)v.w, (double)v.w, ss);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
            if (lane == 0) red[tid >> 6] = ss;
            __syncthreads();
            if (tid == 0) {
                double t = 0.0;
#pragma unroll
                for (int w = 0; w < kGvWaves; ++w) t += red[w];
                inv_sh = (float)(1.0 / sqrt(t / (double)K + (double)eps));
            }
            __syncthreads();
            inv = inv_sh;
        }
    }

    for (int s0 = 0; s0 < NS; s0 += kGvDepth) {
#pragma unroll
        for (int d = 0; d < kGvDepth; ++d) {
            const int sl = s0 + d;
            if (sl < NS) {
                const int i = sl * kGvSlice + lane * 8;
                const int ic = min(i, K - 8);
                float xv[8];
                if constexpr (NORMED) {
                    const float4 a0 = *reinterpret_cast<const float4 *>(a + ic);
                    const float4 a1 = *reinterpret_cast<const float4 *>(a + ic + 4);
                    xv[0] = a0.x * inv; xv[1] = a0.y * inv; xv[2] = a0.z * inv; xv[3] = a0.w * inv;
                    xv[4] = a1.x * inv; xv[5] = a1.y * inv; xv[6] = a1.z * inv; xv[7] = a1.w * inv;
                    if (gamma) {
                        const float4 g0 = *reinterpret_cast<const float4 *>(gamma + ic);
                        const float4 g1 = *reinterpret_cast<const float4 *>(gamma + ic + 4);
                        xv[0] *= g0.x; xv[1] *= g0.y; xv[2] *= g0.z; xv[3] *= g0.w;
                        xv[4] *= g1.x; xv[5] *= g1.y; xv[6] *= g1.z; xv[7] *= g1.w;
                    }
                } else {
                    const u4 xb = *reinterpret_cast<const u4 *>(x + ic);
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        xv[2 * h] = bf16f(xb[h] & 0xffffu);
                        xv[2 * h + 1] = bf16f(xb[h] >> 16);
                    }
                }
                if (i >= K)  // a clamped copy past the row end adds nothing
#pragma unroll
                    for (int h = 0; h < 8; ++h) xv[h] = 0.0f;
#pragma unroll
                for (int q = 0; q < RW; ++q)
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        acc[q] = fmaf(bf16f(buf[d][q][h] & 0xffffu), xv[2 * h], acc[q]);
                        acc[q] = fmaf(bf16f(buf[d][q][h] >> 16), xv[2 * h + 1], acc[q]);
                    }
            }
            load(min(sl + kGvDepth, NS - 1), buf[d]);
        }
    }
#pragma unroll
    for (int q = 0; q < RW; ++q) acc[q] = gv_wave_sum(acc[q]);
}

// z = W_d x for one token, written as the bf16 hi and lo planes the experts read.
template <int RW>
__global__ __launch_bounds__(64 * kGvWaves) void k_gv_down(const uint16_t *__restrict__ W, const uint16_t *__restrict__ x,
                                                           int R, int K, uint16_t *__restrict__ hi,
                                                           uint16_t *__restrict__ lo)
{
    const int lane = threadIdx.x & 63, row0 = (blockIdx.x * kGvWaves + (threadIdx.x >> 6)) * RW;
    float acc[RW];
    gv_rows<RW, false>(W, R, K, row0, x, nullptr, nullptr, false, 0.0f, acc);
#pragma unroll
    for (int q = 0; q < RW; ++q)
        if (lane == q && row0 + q < R) {
            const uint16_t h = bf16_rne(acc[q]);
            hi[row0 + q] = h;
            lo[row0 + q] = bf16_rne(acc[q] - bf16f(h));
        }
}

// out = W_u (RMSNorm(acc) or acc) for one token, then the addend's AS slices
// in order (the shared expert's K-slice partials, stride astride), then the
// epilogue (residual add, bf16 copy) as in k_proj_finish.
template <int RW>
__global__ __launch_bounds__(64 * kGvWaves) void k_gv_up(const uint16_t *__restrict__ W, const float *__restrict__ a,
                                                         const float *__restrict__ gamma, int norm, float eps, int R,
                                                         int K, const float *__restrict__ addend, int AS,
                                                         int64_t astride, float *__restrict__ out, int resid,
                                                         uint16_t *__restrict__ ob)
{
    const int lane = threadIdx.x & 63, row0 = (blockIdx.x * kGvWaves + (threadIdx.x >> 6)) * RW;
    float acc[RW];
    gv_rows<RW, true>(W, R, K, row0, nullptr, a, norm ? gamma : nullptr, norm != 0, eps, acc);
#pragma unroll
    for (int q = 0; q < RW; ++q)
        if (lane == q && row0 + q < R) {
            const int r = row0 + q;
            float v = acc[q];
            if (addend) {
                float ad = addend[r];
                for (int s = 1; s < AS; ++s) ad += addend[(size_t)s * astride + r];
                v += ad;
            }
            if (resid) v = out[r] + v;
            out[r] = v;
            if (ob) ob[r] = bf16_rne(v);
        }
}

constexpr int kGvDownRows = 2;  // rows per wave: R = 3584 gives 448 blocks
constexpr int kGvUpRows = 4;    // R = 7168 gives 448 blocks

// out = W (planes) as fp32 [T][R] (+ addend), or as bf16 hi/lo planes.
static hipError_t launch_proj(const uint16_t *W, const uint16_t *p0, const uint16_t *p1, int T, int R, int Kd,
                              float *part, const float *addend, int AS, float *out, uint16_t *hi, uint16_t *lo,
                              hipStream_t s, const OutEpi &epi = OutEpi())
{
    static const bool lds_set = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_proj<1>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, proj_lds_bytes(1));
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_proj<2>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, proj_lds_bytes(2));
        return true;
    }();
    (void)lds_set;
    const int S = proj_splits(T, R, Kd);
    const int kspan = (Kd / kPjKC + S - 1) / S * kPjKC;
    const dim3 grid((unsigned)((R + kPjRows - 1) / kPjRows), (unsigned)((T + kPjTok - 1) / kPjTok), (unsigned)S);
    if (p1)
        k_proj<2><<<grid, 256, proj_lds_bytes(2), s>>>(W, p0, p1, T, R, Kd, kspan, part);
    else
        k_proj<1><<<grid, 256, proj_lds_bytes(1), s>>>(W, p0, nullptr, T, R, Kd, kspan, part);
    const int64_t n = (int64_t)T * R;
    k_proj_finish<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, S, T, R, addend, AS, out, hi, lo, epi.resid,
                                                                 epi.ob);
    return hipGetLastError();
}

}  // namespace

// K slices of a projection: enough blocks for about 1024 on the chip, each
// slice at least 512 wide, and no empty slice.
int proj_splits(int64_t T, int R, int Kd)
{
    const int64_t blocks = (int64_t)((R + kPjRows - 1) / kPjRows) * ((T + kPjTok - 1) / kPjTok);
    const int64_t want = (1024 + blocks - 1) / blocks;
    const int64_t S = std::max<int64_t>(1, std::min<int64_t>(want, Kd / 512));
    const int kspan = (int)((Kd / kPjKC + S - 1) / S * kPjKC);
    return (Kd + kspan - 1) / kspan;
}

hipError_t launch_latent_forward(const LayerView &L, const uint16_t *x, int T, const int32_t *idx,
                                 const float *w, float *out, char *ws, const WsLayout &lay, hipStream_t s,
                                 Profiler *prof, const OutEpi &epi)
{
    const int Lt = L.Lt;
    uint16_t *zh = reinterpret_cast<uint16_t *>(ws + lay.lat_z), *zl = zh + (size_t)T * Lt;
    float *acc = reinterpret_cast<float *>(ws + lay.lat_acc);
    uint16_t *nh = reinterpret_cast<uint16_t *>(ws + lay.lat_n), *nl = nh + (size_t)T * Lt;
    float *ysh = L.Is > 0 ? reinterpret_cast<float *>(ws + lay.lat_ysh) : nullptr;
    float *part = reinterpret_cast<float *>(ws + lay.lat_part);
    float *ys = reinterpret_cast<float *>(ws + lay.ys);
    hipError_t e;
    const bool one = T == 1;  // one token: the projections as streaming GEMVs
    {
        StageMark m(prof, K3MOE_STAGE_LATENT_IN, s);  // z = Wd x, as bf16 hi and lo
        if (one) {
            const int rpb = kGvWaves * kGvDownRows;
            k_gv_down<kGvDownRows><<<(unsigned)((Lt + rpb - 1) / rpb), 64 * kGvWaves, 0, s>>>(L.lat_down, x, Lt,
                                                                                            L.H, zh, zl);
        } else if ((e = launch_proj(L.lat_down, x, nullptr, T, Lt, L.H, part, nullptr, 1, nullptr, zh, zl, s)) !=
                   hipSuccess) {
            return e;
        }
    }
    int ysh_slices = 1;  // the shared rows' K-slice partials (the streamed form only)
    if (one && latent_t1_ok(L)) {
        // the router slots are the assignments: no permutation, the single-token kernels
        e = launch_latent_t1(L, x, zh, zl, idx, reinterpret_cast<float *>(ws + lay.act),
                             reinterpret_cast<float *>(ws + lay.ash), ws + lay.ys, ysh, s, prof);
    } else {
        launch_perm(L, idx, T, ws, lay, s, prof);
        uint16_t *act_hi = reinterpret_cast<uint16_t *>(ws + lay.act);
        uint16_t *act_lo = act_hi + (size_t)T * L.K * L.I;
        uint16_t *ash_hi = reinterpret_cast<uint16_t *>(ws + lay.ash);
        uint16_t *ash_lo = ash_hi + (size_t)T * L.Is;
        e = launch_grouped(L, x, zh, zl, T, reinterpret_cast<int32_t *>(ws + lay.active_n),
                           reinterpret_cast<int32_t *>(ws + lay.active_e),
                           reinterpret_cast<int32_t *>(ws + lay.active_off), reinterpret_cast<int32_t *>(ws + lay.sorted),
                           act_hi, act_lo, ash_hi, ash_lo, reinterpret_cast<float *>(ws + lay.sh_part),
                           reinterpret_cast<int2 *>(ws + lay.tiles_gu), reinterpret_cast<int2 *>(ws + lay.tiles_dn),
                           reinterpret_cast<int32_t *>(ws + lay.light), reinterpret_cast<int32_t *>(ws + lay.tile_n),
                           ys, ysh, s, prof, term_bufs(ws, lay));
        ysh_slices = stream_shared_ok(L, T) ? stream_shared_down_slices(L.Lt, L.Is, T, L.I) : 1;
    }
    if (e != hipSuccess) return e;
    {
        StageMark m(prof, K3MOE_STAGE_COMBINE, s);  // the routed aggregate [T][L], router order
        launch_combine(L, ys, w, idx, T, Lt, false, acc, s);
    }
    {
        StageMark m(prof, K3MOE_STAGE_LATENT_OUT, s);  // norm, then out = Wu acc (+ shared)
        if (one) {
            const int rpb = kGvWaves * kGvUpRows;
            k_gv_up<kGvUpRows><<<(unsigned)((L.H + rpb - 1) / rpb), 64 * kGvWaves, 0, s>>>(
                L.lat_up, acc, L.lat_norm, L.lat_norm_on, L.lat_eps, L.H, Lt, ysh, ysh_slices, (int64_t)L.H, out,
                epi.resid, epi.ob);
            return hipGetLastError();
        }
        if (L.lat_norm_on)
            k_rms_split<true><<<(unsigned)T, 256, 0, s>>>(acc, Lt, L.lat_norm, L.lat_eps, nh, nl);
        else
            k_rms_split<false><<<(unsigned)T, 256, 0, s>>>(acc, Lt, nullptr, 0.0f, nh, nl);
        if ((e = launch_proj(L.lat_up, nh, nl, T, L.H, Lt, part, ysh, ysh_slices, out, nullptr, nullptr, s, epi)) != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

}  // namespace k3moe
