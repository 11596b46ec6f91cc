// matvec.hip -- batch-1 decode: float-peel PTQ1_0 matvec with the activation
// rotation fused ahead of it, and the reduction epilogues (plain, residual,
// gate/up with SwiGLU).
//
// "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally":
//   - "What Bonsai is": activations are rotated before every folded matmul;
//   - "What Ferrox does with it": each block is read once and its trits are
//     peeled on the float pipeline, floor(3^(n+1) u) - 3 floor(3^n u);
//   - "Speed, and where it goes": gate and up fused into one submission,
//     rotation on the GPU ahead of the matmul it feeds.
//
// Mapping (gfx950): a workgroup owns 256 consecutive output rows and one
// 1024-wide K segment (= one Hadamard chunk = 8 blocks).  Wave 0 rotates the
// segment of x in registers (no LDS butterfly, no barriers inside) and
// parks it in LDS; every lane then owns one output row and streams that
// row's 8 blocks (7 dwords each), reading x as wave-uniform LDS broadcasts.
// Digit sums use sum (d - 1) x = sum d x - sum x, with sum x per block
// precomputed once per workgroup.  Partial sums per (segment, row) are
// reduced by a second kernel in a fixed order (deterministic).
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

// Dot product of one block's 128 trits (bytes in d[0..6]) with xb[0..128),
// before subtracting sum(xb): sum_j digit_j * xb[j].
__device__ __forceinline__ float block_digit_dot(const uint32_t (&d)[kBlockDwords],
                                                 const float *__restrict__ xb)
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kTritBytes; ++i) {
        const float byte = static_cast<float>((d[i >> 2] >> (8 * (i & 3))) & 0xffu);
        const Peel5 p = peel5(byte);
        const int j = kTritsPerByte * i;
        acc = fmaf(p.d0, xb[j + 0], acc);
        acc = fmaf(p.d1, xb[j + 1], acc);
        acc = fmaf(p.d2, xb[j + 2], acc);
        if (j + 3 < kBlockWeights) acc = fmaf(p.d3, xb[j + 3], acc);
        if (j + 4 < kBlockWeights) acc = fmaf(p.d4, xb[j + 4], acc);
    }
    return acc;
}

__global__ void __launch_bounds__(kMvThreads) k_matvec_peel_part(
    const uint8_t *__restrict__ w0, int64_t n0, const uint8_t *__restrict__ w1, int64_t n1,
    int64_t k, const float *__restrict__ x, const float *__restrict__ signs,
    float *__restrict__ part)
{
    __shared__ float xs[kHadamard];
    __shared__ float bsum[kBlocksPerChunk];
    const int tid = threadIdx.x;
    const int64_t rows = n0 + n1;
    const int64_t seg = blockIdx.y;
    const int64_t k0 = seg * kHadamard;
    const int kw = static_cast<int>(k - k0 < kHadamard ? k - k0 : kHadamard);
    const int nblk = kw / kBlockWeights;

    if (signs != nullptr) {  // kw == 1024 (checked by the caller)
        if (tid < kWave) {
            float v[kRotPerLane];
#pragma unroll
            for (int j = 0; j < kRotPerLane; ++j)
                v[j] = x[k0 + tid + kWave * j] * signs[tid + kWave * j];
            fwht1024_wave(v);
#pragma unroll
            for (int j = 0; j < kRotPerLane; ++j) xs[tid + kWave * j] = v[j] * (1.0f / 32.0f);
        }
    } else {
        for (int i = tid; i < kw; i += kMvThreads) xs[i] = x[k0 + i];
    }
    __syncthreads();
    if (tid < nblk) {
        float s = 0.0f;
        for (int j = 0; j < kBlockWeights; ++j) s += xs[tid * kBlockWeights + j];
        bsum[tid] = s;
    }
    __syncthreads();

    const int64_t r = static_cast<int64_t>(blockIdx.x) * kMvRowsPerWg + tid;
    if (r >= rows) return;
    const int64_t pitch = (k / kBlockWeights) * kBlockBytes;
    const uint8_t *wrow = (r < n0) ? (w0 + r * pitch) : (w1 + (r - n0) * pitch);
    const uint32_t *bp =
        reinterpret_cast<const uint32_t *>(wrow + (k0 / kBlockWeights) * kBlockBytes);

    float out = 0.0f;
    if (nblk == kBlocksPerChunk) {
        uint32_t d[kBlocksPerChunk][kBlockDwords];
#pragma unroll
        for (int b = 0; b < kBlocksPerChunk; ++b)
#pragma unroll
            for (int q = 0; q < kBlockDwords; ++q) d[b][q] = bp[b * kBlockDwords + q];
#pragma unroll
        for (int b = 0; b < kBlocksPerChunk; ++b) {
            const float acc = block_digit_dot(d[b], xs + b * kBlockWeights);
            const float sc = half_bits_to_float(d[b][kBlockDwords - 1] >> 16);
            out = fmaf(sc, acc - bsum[b], out);
        }
    } else {
        for (int b = 0; b < nblk; ++b) {
            uint32_t d[kBlockDwords];
#pragma unroll
            for (int q = 0; q < kBlockDwords; ++q) d[q] = bp[b * kBlockDwords + q];
            const float acc = block_digit_dot(d, xs + b * kBlockWeights);
            const float sc = half_bits_to_float(d[kBlockDwords - 1] >> 16);
            out = fmaf(sc, acc - bsum[b], out);
        }
    }
    part[seg * rows + r] = out;
}

__global__ void __launch_bounds__(kEwThreads) k_reduce_rows(const float *__restrict__ part,
                                                            int64_t n, int64_t nseg,
                                                            const float *residual, float *y)
{
    const int64_t r = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x;
    if (r >= n) return;
    float s = 0.0f;
    for (int64_t q = 0; q < nseg; ++q) s += part[q * n + r];
    y[r] = residual ? residual[r] + s : s;
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// Sum of squares of x[0..d) across the workgroup (every thread gets it).
__device__ float block_sum_squares(const float *__restrict__ x, int64_t d)
{
    __shared__ float red[kEwThreads / kWave];
    float s = 0.0f;
    for (int64_t i = threadIdx.x; i < d; i += kEwThreads) s = fmaf(x[i], x[i], s);
#pragma unroll
    for (int h = kWave / 2; h > 0; h >>= 1) s += __shfl_xor(s, h, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kEwThreads / kWave; ++w) t += red[w];
    return t;
}

__global__ void __launch_bounds__(kEwThreads) k_reduce_gate_up(
    const float *__restrict__ part, int64_t f, int64_t nseg, float *__restrict__ g,
    float *__restrict__ u, float *__restrict__ h, const float *__restrict__ x_rms, int64_t d,
    float rms_eps)
{
    float a = 1.0f;
    if (x_rms != nullptr) a = 1.0f / sqrtf(block_sum_squares(x_rms, d) / static_cast<float>(d) + rms_eps);
    const int64_t r = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x;
    if (r >= f) return;
    float sg = 0.0f, su = 0.0f;
    for (int64_t q = 0; q < nseg; ++q) {
        sg += part[q * 2 * f + r];
        su += part[q * 2 * f + f + r];
    }
    sg *= a;
    su *= a;
    if (g) g[r] = sg;
    if (u) u[r] = su;
    if (h) h[r] = silu_mul(sg, su);
}

__global__ void __launch_bounds__(kEwThreads) k_swiglu(const float *g, const float *u, float *h,
                                                       int64_t len)
{
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x; i < len;
         i += static_cast<int64_t>(gridDim.x) * kEwThreads)
        h[i] = silu_mul(g[i], u[i]);
}

size_t matvec_part_floats(int64_t rows, int64_t k)
{
    const int64_t nseg = (k + kHadamard - 1) / kHadamard;
    return static_cast<size_t>(rows * nseg);
}

hipError_t launch_matvec_part(const uint8_t *w0, int64_t n0, const uint8_t *w1, int64_t n1,
                              int64_t k, const float *x, const float *signs, float *part,
                              hipStream_t s)
{
    const int64_t rows = n0 + n1;
    const int64_t nseg = (k + kHadamard - 1) / kHadamard;
    if (rows == 0 || nseg == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((rows + kMvRowsPerWg - 1) / kMvRowsPerWg),
                    static_cast<unsigned>(nseg));
    hipLaunchKernelGGL(k_matvec_peel_part, grid, dim3(kMvThreads), 0, s, w0, n0, w1, n1, k, x,
                       signs, part);
    return hipGetLastError();
}

hipError_t launch_reduce_rows(const float *part, int64_t n, int64_t nseg, const float *residual,
                              float *y, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_reduce_rows, dim3(static_cast<unsigned>((n + kEwThreads - 1) / kEwThreads)),
                       dim3(kEwThreads), 0, s, part, n, nseg, residual, y);
    return hipGetLastError();
}

hipError_t launch_reduce_gate_up(const float *part, int64_t f, int64_t nseg, float *g, float *u,
                                 float *h, const float *x_rms, int64_t d, float rms_eps,
                                 hipStream_t s)
{
    if (f == 0) return hipSuccess;
    hipLaunchKernelGGL(k_reduce_gate_up,
                       dim3(static_cast<unsigned>((f + kEwThreads - 1) / kEwThreads)),
                       dim3(kEwThreads), 0, s, part, f, nseg, g, u, h, x_rms, d, rms_eps);
    return hipGetLastError();
}

hipError_t launch_swiglu(const float *g, const float *u, float *h, int64_t len, hipStream_t s)
{
    if (len == 0) return hipSuccess;
    int64_t blocks = (len + kEwThreads - 1) / kEwThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_swiglu, dim3(static_cast<unsigned>(blocks)), dim3(kEwThreads), 0, s, g, u,
                       h, len);
    return hipGetLastError();
}

}  // namespace ptq1
