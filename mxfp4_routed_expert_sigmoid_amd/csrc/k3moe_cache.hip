// Experts beyond HBM: an HBM arena of expert slots fed from host memory.
//
// Policy (the "kimi-k3-in-c" README, §12 "An LRU cache for the experts"): a
// slot is empty, reserved for an expert being read, or holding an expert;
// misses take an empty slot when there is one, else the least recently used
// slot that is neither reserved nor pinned; slots are reserved one request at
// a time so no two experts take the same slot, the experts are read, and only
// then published. From the Kimi-K3.cpp README ("The consumer-memory idea"):
// every hit of the step is pinned before any victim is chosen, and the
// results are reduced in router order whatever order the reads finish in.
//
// Here the whole policy runs on the device, in stream order, so a step needs
// no host round trip:
//   k_cache_plan  one block: the slot table is loaded into LDS, the step's
//                 distinct experts are listed in order of first appearance
//                 in the (token, slot) assignments, hits are pinned and
//                 stamped, then one wave reserves a victim per miss in
//                 request order (a wave-wide minimum over the slots' keys:
//                 empty slots first by index, then least recently used,
//                 ties by index; pinned and reserved slots never qualify).
//                 It writes the fill list, the assignments' slot ids (-1:
//                 invalid id, or no slot left) and the table back.
//   k_cache_fill  copies each listed expert's six tensors from host memory
//                 (device-visible pinned pages, read over the host link)
//                 into its slot.
// The expert kernels then run on the arena with slot ids in place of expert
// ids: the same bytes through the same kernels, combined in router order.
#include "k3moe_internal.h"

namespace k3moe {
namespace {

typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 1024;
constexpr int kFillThreads = 256;
constexpr int kFillQ = 8;  // 16-byte loads in flight per thread

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m)
{
    const int lo = __shfl_xor((int)(uint32_t)v, m), hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        const unsigned long long o = shfl_xor_u64(v, m);
        v = o < v ? o : v;
    }
    return v;
}

// Victim order of slot s: empty slots first by index, then by last use and
// index; pinned or reserved (this step) slots never qualify.
__device__ __forceinline__ unsigned long long victim_key(int s, const int *key_of, const long long *used_at,
                                                        const uint8_t *pinned)
{
    if (pinned[s]) return ~0ull;
    if (key_of[s] < 0) return (unsigned long long)s;
    return (1ull << 62) | ((unsigned long long)used_at[s] << kCacheSlotBits) | (unsigned long long)s;
}

__global__ __launch_bounds__(kPlanThreads) void k_cache_plan(CachePlanParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int E = p.E, S = p.S;
    long long *used_at = reinterpret_cast<long long *>(lds);  // [S]
    int *first = reinterpret_cast<int *>(used_at + S);        // [E] first assignment of each expert
    int *slot_of = first + E;                                 // [E] slot of each expert, -1: none
    int *req = slot_of + E;                                   // [E] requests in order
    int *key_of = req + E;                                    // [S] expert in each slot, -1: empty
    uint8_t *pinned = reinterpret_cast<uint8_t *>(key_of + S);  // [S] pinned or reserved this step
    __shared__ int wtot[kPlanThreads / 64];
    __shared__ int nreq_sh, chunk_sh;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    for (int e = tid; e < E; e += kPlanThreads) {
        first[e] = 0x7fffffff;
        slot_of[e] = p.slot_of[e];
    }
    for (int s = tid; s < S; s += kPlanThreads) {
        key_of[s] = p.key_of[s];
        used_at[s] = p.used_at[s];
        pinned[s] = 0;
    }
    if (tid == 0) nreq_sh = 0;
    __syncthreads();
    for (int64_t a = tid; a < p.n; a += kPlanThreads) {
        const int e = p.idx[a];
        if (e >= 0 && e < E) atomicMin(&first[e], (int)a);
    }
    __syncthreads();

    // the distinct experts in order of first appearance (ordered compaction)
    for (int64_t c0 = 0; c0 < p.n; c0 += kPlanThreads) {
        const int64_t a = c0 + tid;
        const int e = a < p.n ? p.idx[a] : -1;
        const bool f = a < p.n && e >= 0 && e < E && first[e] == (int)a;
        const uint64_t m = __ballot(f);
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (lane == 0) wtot[wv] = __popcll(m);
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int w = 0; w < kPlanThreads / 64; ++w) {
                const int c = wtot[w];
                wtot[w] = run;
                run += c;
            }
            chunk_sh = run;
        }
        __syncthreads();
        if (f) req[nreq_sh + wtot[wv] + below] = e;
        __syncthreads();
        if (tid == 0) nreq_sh += chunk_sh;
        __syncthreads();
    }
    const int nreq = nreq_sh;
    const long long tick0 = (long long)p.ctr[kCtrTick];

    // hits: pinned, stamped with their request position
    for (int r = tid; r < nreq; r += kPlanThreads) {
        const int s = slot_of[req[r]];
        if (s >= 0) {
            pinned[s] = 1;
            used_at[s] = tick0 + r + 1;
        }
    }
    __syncthreads();

    // misses: one victim each, in request order (wave 0; each lane owns the
    // slots lane, lane + 64, ... and keeps its best key)
    if (wv == 0) {
        unsigned long long best = ~0ull;
        auto rescan = [&]() {
            best = ~0ull;
            for (int s = lane; s < S; s += 64) {
                const unsigned long long k = victim_key(s, key_of, used_at, pinned);
                best = k < best ? k : best;
            }
        };
        rescan();
        int nfill = 0;
        unsigned long long misses = 0, evict = 0, drops = 0;
        for (int r = 0; r < nreq; ++r) {
            const int e = req[r];
            if (slot_of[e] >= 0) continue;  // a hit (every lane reads the same word)
            const unsigned long long m = wave_min_u64(best);
            if (m == ~0ull) {  // every slot pinned or reserved: the request goes without
                ++drops;
                continue;
            }
            const int s = (int)(m & ((1ull << kCacheSlotBits) - 1));
            const int old = key_of[s];
            if (old >= 0) ++evict;
            ++misses;
            if (lane == (s & 63)) {
                if (old >= 0) slot_of[old] = -1;
                key_of[s] = e;
                slot_of[e] = s;
                used_at[s] = tick0 + r + 1;
                pinned[s] = 1;
                p.fill[nfill] = make_int2(e, s);
                rescan();
            }
            ++nfill;
        }
        if (lane == 0) {
            *p.nfill = nfill;
            p.ctr[kCtrTick] += (unsigned long long)nreq;
            p.ctr[kCtrSteps] += 1;
            p.ctr[kCtrRequests] += (unsigned long long)nreq;
            p.ctr[kCtrHits] += (unsigned long long)nreq - misses - drops;
            p.ctr[kCtrMisses] += misses;
            p.ctr[kCtrEvictions] += evict;
            p.ctr[kCtrDropped] += drops;
            p.ctr[kCtrBytes] += misses * (unsigned long long)p.expert_bytes;
        }
    }
    __syncthreads();

    for (int64_t a = tid; a < p.n; a += kPlanThreads) {
        const int e = p.idx[a];
        p.remap[a] = (e >= 0 && e < E) ? slot_of[e] : -1;
    }
    for (int e = tid; e < E; e += kPlanThreads) p.slot_of[e] = slot_of[e];
    for (int s = tid; s < S; s += kPlanThreads) {
        p.key_of[s] = key_of[s];
        p.used_at[s] = used_at[s];
    }
}

// Block b copies bytes [c * kFillChunk, ...) of fill entry f = b / nchunk
// (c = b % nchunk) of the expert's six tensors, seen as one run of
// expert_bytes (segment i: seg_len[i] bytes, from src[i] + e * src_stride[i]
// to the slot's offset seg_off[i]). Every length and offset is a multiple of
// 16 bytes.
__global__ __launch_bounds__(kFillThreads) void k_cache_fill(CacheFillParams p)
{
    const int f = blockIdx.x / p.nchunk, c = blockIdx.x - f * p.nchunk;
    if (f >= *p.nfill) return;
    const int2 es = p.fill[f];
    const int64_t lo = (int64_t)c * kFillChunk;
    const int64_t hi = lo + kFillChunk < p.expert_bytes ? lo + kFillChunk : p.expert_bytes;
    int64_t base = 0;
    for (int i = 0; i < 6; ++i) {
        const int64_t a = lo > base ? lo : base;
        const int64_t b = hi < base + p.seg_len[i] ? hi : base + p.seg_len[i];
        if (a < b) {
            const u4 *src = reinterpret_cast<const u4 *>(p.src[i] + (int64_t)es.x * p.src_stride[i] + (a - base));
            u4 *dst = reinterpret_cast<u4 *>(p.arena + (int64_t)es.y * p.slot_bytes + p.seg_off[i] + (a - base));
            const int64_t n = (b - a) / 16;
            for (int64_t v0 = 0; v0 < n; v0 += (int64_t)kFillThreads * kFillQ) {
                u4 t[kFillQ];
#pragma unroll
                for (int q = 0; q < kFillQ; ++q) {
                    const int64_t v = v0 + threadIdx.x + (int64_t)q * kFillThreads;
                    if (v < n) t[q] = src[v];
                }
#pragma unroll
                for (int q = 0; q < kFillQ; ++q) {
                    const int64_t v = v0 + threadIdx.x + (int64_t)q * kFillThreads;
                    if (v < n) dst[v] = t[q];
                }
            }
        }
        base += p.seg_len[i];
    }
}

// Every slot empty, counters zero.
__global__ void k_cache_init(unsigned long long *ctr, int32_t *slot_of, int E, int32_t *key_of,
                             long long *used_at, int S)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < kCtrCount) ctr[i] = 0ull;
    if (i < E) slot_of[i] = -1;
    if (i < S) {
        key_of[i] = -1;
        used_at[i] = 0;
    }
}

}  // namespace

size_t cache_plan_lds_bytes(int E, int S) { return (size_t)S * 8 + (size_t)E * 12 + (size_t)S * 4 + S; }

hipError_t launch_cache_init(unsigned long long *ctr, int32_t *slot_of, int E, int32_t *key_of, long long *used_at,
                             int S, hipStream_t s)
{
    const int n = std::max(std::max(E, S), (int)kCtrCount);
    k_cache_init<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(ctr, slot_of, E, key_of, used_at, S);
    return hipGetLastError();
}

hipError_t launch_cache_plan_fill(const CachePlanParams &pp, const CacheFillParams &fp, int max_fill,
                                  hipStream_t s, Profiler *prof)
{
    static const bool lds_set = [] {
        // the largest table (the kernel's static LDS comes on top)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_cache_plan),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)cache_plan_lds_bytes(kMaxExperts, kMaxExperts));
        return true;
    }();
    (void)lds_set;
    {
        StageMark m(prof, K3MOE_STAGE_CACHE_PLAN, s);
        k_cache_plan<<<1, kPlanThreads, cache_plan_lds_bytes(pp.E, pp.S), s>>>(pp);
    }
    if (max_fill > 0) {
        StageMark m(prof, K3MOE_STAGE_CACHE_FILL, s);
        k_cache_fill<<<(unsigned)((int64_t)max_fill * fp.nchunk), kFillThreads, 0, s>>>(fp);
    }
    return hipGetLastError();
}

}  // namespace k3moe
