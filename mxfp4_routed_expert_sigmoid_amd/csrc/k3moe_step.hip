// The pre-MoE norm of a decoder layer: the layer's input is the RMSNorm of
// the residual stream with the post-attention gain (the "kimi-k3-in-c"
// README, the decoder-layer listing after "Aggregate, attend, aggregate
// again": hin = k3_rmsnorm(h, post_norm) feeds k3_moe), in the exact form of
// §5 "Kernels with a floating point contract" (k3_rmsnorm): the sum of
// squares in fp64, epsilon inside the root, inv = (float)(1 / sqrt(ss / n +
// eps)), then x * inv * gain as two fp32 products. The expert layer takes
// bf16 tokens, so the normed value is rounded once, to nearest even.
#include "k3moe_device.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kPnThreads = 256;
constexpr int kPnV = 8;  // float4 loads in flight per thread and pass (rows up to 8192 in one pass)

__device__ __forceinline__ uint32_t pn_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One block per token; n % 4 == 0. A row of at most kPnThreads * kPnV float4
// (n <= 8192) is read once: the gain is loaded beside it and both stay in
// registers across the reduction, so the only memory latency before the
// stores is the first one.
__global__ __launch_bounds__(kPnThreads) void k_prenorm(const float *__restrict__ h, int n,
                                                        const float *__restrict__ gamma, float eps,
                                                        uint16_t *__restrict__ x)
{
    __shared__ double red[kPnThreads / 64];
    __shared__ float inv_sh;
    const int t = blockIdx.x, tid = threadIdx.x, nv = n / 4;
    const float4 *a = reinterpret_cast<const float4 *>(h + (size_t)t * n);
    const float4 *gm = reinterpret_cast<const float4 *>(gamma);
    const bool one = nv <= kPnThreads * kPnV;
    float4 v1[kPnV], g1[kPnV];
    double ss = 0.0;
    if (one) {
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            const int i = min(tid + kPnThreads * j, nv - 1);
            v1[j] = a[i];
            g1[j] = gm[i];
        }
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            if (tid + kPnThreads * j >= nv) v1[j] = float4{0.0f, 0.0f, 0.0f, 0.0f};
            ss = fma((double)v1[j].x, (double)v1[j].x, ss);
            ss = fma((double)v1[j].y, (double)v1[j].y, ss);
            ss = fma((double)v1[j].z, (double)v1[j].z, ss);
            ss = fma((double)v1[j].w, (double)v1[j].w, ss);
        }
    }
    for (int c0 = 0; !one && c0 < nv; c0 += kPnThreads * kPnV) {
        float4 v[kPnV];
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            const int i = c0 + tid + kPnThreads * j;
            v[j] = i < nv ? a[i] : float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
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
    if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int q = 0; q < kPnThreads / 64; ++q) tot += red[q];
        inv_sh = (float)(1.0 / sqrt(tot / (double)n + (double)eps));
    }
    __syncthreads();
    const float inv = inv_sh;
    uint2 *xo = reinterpret_cast<uint2 *>(x + (size_t)t * n);
    if (one) {
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            const int i = tid + kPnThreads * j;
            if (i < nv)
                xo[i] = uint2{pn_bf16(v1[j].x * inv * g1[j].x) | (pn_bf16(v1[j].y * inv * g1[j].y) << 16),
                              pn_bf16(v1[j].z * inv * g1[j].z) | (pn_bf16(v1[j].w * inv * g1[j].w) << 16)};
        }
    }
    for (int c0 = 0; !one && c0 < nv; c0 += kPnThreads * kPnV) {
        float4 v[kPnV], g[kPnV];
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            const int i = min(c0 + tid + kPnThreads * j, nv - 1);
            v[j] = a[i];
            g[j] = gm[i];
        }
#pragma unroll
        for (int j = 0; j < kPnV; ++j) {
            const int i = c0 + tid + kPnThreads * j;
            if (i < nv)
                xo[i] = uint2{pn_bf16(v[j].x * inv * g[j].x) | (pn_bf16(v[j].y * inv * g[j].y) << 16),
                              pn_bf16(v[j].z * inv * g[j].z) | (pn_bf16(v[j].w * inv * g[j].w) << 16)};
        }
    }
}


// The step's pre-MoE norm and the one-token router in one launch (T = 1):
// every block normalises the residual row itself — the same fp64 sum in the
// same order as k_prenorm, so every block gets the same inv and the same
// bf16 token — keeps the token in LDS for its four router rows (one wave
// each, as k_router: exact bf16 products summed in fp64, slices of 512 in
// order, a fixed-order butterfly) and block 0 stores it for the expert
// kernels. The router rows are loaded first: their latency overlaps the
// norm's. n <= 8192, n % 8 == 0.
constexpr int kPrSl = 16;  // 512-element router slices per lane (n <= 8192)

__global__ __launch_bounds__(kPnThreads) void k_prenorm_router(const float *__restrict__ h, int n,
                                                               const float *__restrict__ gamma, float eps,
                                                               const uint16_t *__restrict__ Wr,
                                                               const float *__restrict__ bias, int E,
                                                               uint16_t *__restrict__ x, float *__restrict__ sc,
                                                               float *__restrict__ ch)
{
    static_assert(kPnThreads == 256, "four router rows per block");
    __shared__ u4 x_l[8192 / 8];
    __shared__ double red[kPnThreads / 64];
    __shared__ float inv_sh;
    const int tid = threadIdx.x, lane = tid & 63, nv = n / 4;
    const int e = blockIdx.x * 4 + (tid >> 6);
    const uint16_t *wr = Wr + (size_t)min(e, E - 1) * n;
    u4 wv[kPrSl];
#pragma unroll
    for (int c = 0; c < kPrSl; ++c) {
        const int i = 8 * lane + 512 * c;
        wv[c] = i < n ? ld16_stream(wr + i) : u4{0u, 0u, 0u, 0u};
    }
    const float4 *a = reinterpret_cast<const float4 *>(h);
    const float4 *gm = reinterpret_cast<const float4 *>(gamma);
    float4 v1[kPnV], g1[kPnV];
#pragma unroll
    for (int j = 0; j < kPnV; ++j) {
        const int i = min(tid + kPnThreads * j, nv - 1);
        v1[j] = a[i];
        g1[j] = gm[i];
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kPnV; ++j) {
        if (tid + kPnThreads * j >= nv) v1[j] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        ss = fma((double)v1[j].x, (double)v1[j].x, ss);
        ss = fma((double)v1[j].y, (double)v1[j].y, ss);
        ss = fma((double)v1[j].z, (double)v1[j].z, ss);
        ss = fma((double)v1[j].w, (double)v1[j].w, ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int q = 0; q < kPnThreads / 64; ++q) tot += red[q];
        inv_sh = (float)(1.0 / sqrt(tot / (double)n + (double)eps));
    }
    __syncthreads();
    const float inv = inv_sh;
    uint2 *xl = reinterpret_cast<uint2 *>(x_l);
#pragma unroll
    for (int j = 0; j < kPnV; ++j) {
        const int i = tid + kPnThreads * j;
        if (i < nv) {
            const uint2 q = uint2{pn_bf16(v1[j].x * inv * g1[j].x) | (pn_bf16(v1[j].y * inv * g1[j].y) << 16),
                                  pn_bf16(v1[j].z * inv * g1[j].z) | (pn_bf16(v1[j].w * inv * g1[j].w) << 16)};
            xl[i] = q;
            if (blockIdx.x == 0) reinterpret_cast<uint2 *>(x)[i] = q;
        }
    }
    __syncthreads();
    if (e >= E) return;
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < kPrSl; ++c) {
        const int i = 8 * lane + 512 * c;
        const u4 xv = i < n ? x_l[i / 8] : u4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = fma((double)bf16f(wv[c][q] & 0xffffu), (double)bf16f(xv[q] & 0xffffu), acc);
            acc = fma((double)bf16f(wv[c][q] >> 16), (double)bf16f(xv[q] >> 16), acc);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) router_finish(acc, 0, e, E, bias, sc, ch, nullptr);
}

}  // namespace

hipError_t launch_prenorm(const float *h, int T, int H, const float *gamma, float eps, uint16_t *x, hipStream_t s)
{
    k_prenorm<<<(unsigned)T, kPnThreads, 0, s>>>(h, H, gamma, eps, x);
    return hipGetLastError();
}

bool prenorm_router_ok(const LayerView &L) { return L.H <= 8192 && L.H % 8 == 0; }

hipError_t launch_prenorm_router(const LayerView &L, const float *h, const float *gamma, float eps, uint16_t *x,
                                 float *sc, float *ch, hipStream_t s)
{
    k_prenorm_router<<<(unsigned)((L.E + 3) / 4), kPnThreads, 0, s>>>(h, L.H, gamma, eps, L.router_w,
                                                                    L.router_bias, L.E, x, sc, ch);
    return hipGetLastError();
}

}  // namespace k3moe
