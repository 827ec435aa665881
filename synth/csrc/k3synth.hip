// Device side of the seeded input generators: the splitmix64 output function
// (S. Vigna, public domain) over a counter, word i of stream k being
// mix64(k + (i + 1) * 0x9E3779B97F4A7C15). Generates MXFP4 nibbles and E8M0
// scale bytes in HBM; holds none of the layer's arithmetic.
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__global__ void k_fill_words(uint64_t *dst, int64_t nwords, uint64_t key, int64_t start_word)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = mix64(key + (uint64_t)(start_word + i + 1) * kGamma);
}

__global__ void k_fill_scales(uint8_t *dst, int64_t n, uint64_t key, int64_t start, int lo, int span)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = (uint8_t)(lo + mix64(key + (uint64_t)(start + i + 1) * kGamma) % (uint64_t)span);
}

// Reads every 16-byte word of a buffer once (a calibration kernel of known
// traffic for hardware byte counters); writes one word only if the xor of the
// data hits a fixed value.
__global__ void k_read_probe(const uint4 *src, int64_t n16, unsigned *sink)
{
    unsigned acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

unsigned grid_for(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); }

}  // namespace

extern "C" {

// Bytes [start, start + nbytes) of a packed-nibble stream; start, nbytes and
// dst must be multiples of 8. Returns 0, or -1 on bad arguments, -2 on a HIP
// error.
int k3synth_fill_packed(void *dst, int64_t nbytes, uint64_t key, int64_t start, void *stream)
{
    if (!dst || nbytes < 0 || start < 0 || (nbytes | start) % 8 || (uintptr_t)dst % 8) return -1;
    if (nbytes == 0) return 0;
    k_fill_words<<<grid_for(nbytes / 8), 256, 0, (hipStream_t)stream>>>((uint64_t *)dst, nbytes / 8, key,
                                                                         start / 8);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Entries [start, start + n) of a scale stream: lo + (word mod span).
int k3synth_fill_scales(void *dst, int64_t n, uint64_t key, int64_t start, int lo, int span, void *stream)
{
    if (!dst || n < 0 || start < 0 || span <= 0 || lo < 0 || lo + span > 256) return -1;
    if (n == 0) return 0;
    k_fill_scales<<<grid_for(n), 256, 0, (hipStream_t)stream>>>((uint8_t *)dst, n, key, start, lo, span);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Launch the read-probe over nbytes (a multiple of 16) of src; sink is a
// 4-byte device word.
int k3synth_read_probe(const void *src, int64_t nbytes, void *sink, void *stream)
{
    if (!src || !sink || nbytes < 0 || nbytes % 16 || (uintptr_t)src % 16) return -1;
    k_read_probe<<<4096, 256, 0, (hipStream_t)stream>>>((const uint4 *)src, nbytes / 16, (unsigned *)sink);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
