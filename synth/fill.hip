// fill.hip -- device implementation of the seeded input generator defined in
// synth/__init__.py (counter-based SplitMix64: Steele, Lea & Flood 2014).
// Test and bench infrastructure: it produces raw inputs only and holds none
// of the method's arithmetic.  Element i of a stream is
//   mix64(key + (i + 1) * 0x9E3779B97F4A7C15),  key computed on the host.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, int64_t i)
{
    return mix64(key + static_cast<uint64_t>(i + 1) * 0x9E3779B97F4A7C15ull);
}

constexpr uint64_t kT1 = 2702159776422297ull;  // int(0.3 * 2^53)
constexpr uint64_t kT2 = 6305039478318694ull;  // int(0.7 * 2^53)

__global__ void k_trits(int8_t *out, uint64_t key, int64_t start, int64_t count)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < count;
         t += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t r = draw(key, start + t) >> 11;
        out[t] = r < kT1 ? int8_t(-1) : (r < kT2 ? int8_t(0) : int8_t(1));
    }
}

__global__ void k_table16(uint16_t *out, const uint16_t *table, uint64_t key, int64_t start, int64_t count)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < count;
         t += (int64_t)gridDim.x * blockDim.x)
        out[t] = table[draw(key, start + t) >> 48];
}

__global__ void k_table32(float *out, const float *table, uint64_t key, int64_t start, int64_t count)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < count;
         t += (int64_t)gridDim.x * blockDim.x)
        out[t] = table[draw(key, start + t) >> 48];
}

unsigned grid(int64_t count)
{
    int64_t g = (count + 255) / 256;
    return static_cast<unsigned>(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

extern "C" {

int synth_fill_trits(int8_t *out, uint64_t key, int64_t start, int64_t count, hipStream_t s)
{
    if (count <= 0) return 0;
    hipLaunchKernelGGL(k_trits, dim3(grid(count)), dim3(256), 0, s, out, key, start, count);
    return static_cast<int>(hipGetLastError());
}

int synth_fill_table16(uint16_t *out, const uint16_t *table, uint64_t key, int64_t start, int64_t count,
                       hipStream_t s)
{
    if (count <= 0) return 0;
    hipLaunchKernelGGL(k_table16, dim3(grid(count)), dim3(256), 0, s, out, table, key, start, count);
    return static_cast<int>(hipGetLastError());
}

int synth_fill_table32(float *out, const float *table, uint64_t key, int64_t start, int64_t count,
                       hipStream_t s)
{
    if (count <= 0) return 0;
    hipLaunchKernelGGL(k_table32, dim3(grid(count)), dim3(256), 0, s, out, table, key, start, count);
    return static_cast<int>(hipGetLastError());
}

}
