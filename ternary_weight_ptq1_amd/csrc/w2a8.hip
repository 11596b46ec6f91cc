// w2a8.hip -- the 8-bit-activation decode matvec ("Why I Am Building Another
// Inference Engine", Level 5: integer kernels pair ternary weights with
// int8 activations, the numerics BitNet b1.58 was trained with; Level 4: a
// BitNet layer rounds its activations to int8 ahead of its ternary matmuls).
//
// x [k] -> q = rint(x * c) with c = float(127 / max|x|) (c = 0 when x is all
// zeros), integers in [-127, 127] held as fp32; the lookup-table matvec then
// sums trits times q exactly (every table entry and every per-block sum is an
// integer below 2^24, so fp32 adds are exact) and scales each block by its
// fp16 scale; the sum kernel below adds the slices and multiplies by the
// dequantisation step max|x| / 127.
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

constexpr int kQThreads = 1024;
constexpr int kQPer = 24;  // values per thread held in registers (k <= 24576 in one pass)
constexpr int kSumBatch = 72;  // slices loaded at once (all of them up to K = 18432)

// One workgroup: max |x| over k, then q and the step.  Every load of the
// first kQPer x 1024 values is requested before the reduction (clamped
// addresses); longer vectors loop over the rest.
__global__ void __launch_bounds__(kQThreads) k_w2a8_quant(const float *__restrict__ x, int64_t k,
                                                          float *__restrict__ q, float *__restrict__ step)
{
    __shared__ float red[kQThreads / kWave];
    const int tid = threadIdx.x;
    float v[kQPer];
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
        const int64_t i = tid + static_cast<int64_t>(kQThreads) * j;
        v[j] = x[i < k ? i : k - 1];
    }
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) mx = fmaxf(mx, fabsf(v[j]));  // clamped copies repeat x[k - 1]
    for (int64_t i = tid + static_cast<int64_t>(kQThreads) * kQPer; i < k; i += kQThreads) mx = fmaxf(mx, fabsf(x[i]));
#pragma unroll
    for (int h = kWave / 2; h > 0; h >>= 1) mx = fmaxf(mx, __shfl_xor(mx, h, kWave));
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = mx;
    __syncthreads();
    float g = 0.0f;
#pragma unroll
    for (int w = 0; w < kQThreads / kWave; ++w) g = fmaxf(g, red[w]);
    // the multiplier rounded once from its exact quotient (double division
    // is correctly rounded; the conversion rounds to nearest)
    const float c = g > 0.0f ? static_cast<float>(127.0 / static_cast<double>(g)) : 0.0f;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
        const int64_t i = tid + static_cast<int64_t>(kQThreads) * j;
        if (i < k) q[i] = rintf(v[j] * c);
    }
    for (int64_t i = tid + static_cast<int64_t>(kQThreads) * kQPer; i < k; i += kQThreads) q[i] = rintf(x[i] * c);
    if (tid == 0) step[0] = static_cast<float>(static_cast<double>(g) / 127.0);
}

// y[r] = (residual ? residual[r] : 0) + step * sum_s part[s][r], slices in
// order, loaded kSumBatch slices at a time.
__global__ void __launch_bounds__(kEwThreads) k_w2a8_sum(const float *__restrict__ part, int64_t n, int ns,
                                                         const float *__restrict__ step,
                                                         const float *__restrict__ residual, float *__restrict__ y)
{
    const int64_t r0 = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x;
    const int64_t r = r0 < n ? r0 : n - 1;  // clamped: the loads stay uniform
    const float st = step[0];
    const float res = residual != nullptr ? residual[r] : 0.0f;
    float t = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += kSumBatch) {
        float b[kSumBatch];
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j) {
            const int sj = s0 + j < ns ? s0 + j : ns - 1;
            b[j] = part[static_cast<int64_t>(sj) * n + r];
        }
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j)
            if (s0 + j < ns) t += b[j];
    }
    if (r0 < n) y[r] = residual != nullptr ? fmaf(st, t, res) : st * t;
}

// y [m][n] *= step[row]
__global__ void __launch_bounds__(kEwThreads) k_w2a8_scale_rows(float *__restrict__ y, int64_t m, int64_t n,
                                                                const float *__restrict__ step)
{
    const int64_t i = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x;
    if (i >= m * n) return;
    y[i] *= step[i / n];
}

hipError_t launch_w2a8_scale_rows(float *y, int64_t m, int64_t n, const float *step, hipStream_t s)
{
    const int64_t total = m * n;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_w2a8_scale_rows, dim3(static_cast<unsigned>((total + kEwThreads - 1) / kEwThreads)),
                       dim3(kEwThreads), 0, s, y, m, n, step);
    return hipGetLastError();
}

hipError_t launch_w2a8_quant(const float *x, int64_t k, float *q, float *step, hipStream_t s)
{
    if (k == 0) return hipSuccess;
    hipLaunchKernelGGL(k_w2a8_quant, dim3(1), dim3(kQThreads), 0, s, x, k, q, step);
    return hipGetLastError();
}

hipError_t launch_w2a8_sum(const float *part, int64_t n, int64_t k, const float *step, const float *residual,
                           float *y, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const int ns = static_cast<int>(lut_nslices(k));
    hipLaunchKernelGGL(k_w2a8_sum, dim3(static_cast<unsigned>((n + kEwThreads - 1) / kEwThreads)), dim3(kEwThreads),
                       0, s, part, n, ns, step, residual, y);
    return hipGetLastError();
}

}  // namespace ptq1
