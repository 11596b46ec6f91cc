// w2a8.hip -- the 8-bit-activation decode matvec ("Why I Am Building Another
// Inference Engine", Level 5: the fast kernels multiply the ternary weights
// with 8-bit integer activations, which is the model BitNet b1.58 was trained
// as; Level 4's BitNet layer quantises its activations before the ternary
// projections).
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

// One workgroup: max |x| over k, then q and the step.
__global__ void __launch_bounds__(kQThreads) k_w2a8_quant(const float *__restrict__ x, int64_t k,
                                                          float *__restrict__ q, float *__restrict__ step)
{
    __shared__ float red[kQThreads / kWave];
    const int tid = threadIdx.x;
    float mx = 0.0f;
    for (int64_t i = tid; i < k; i += kQThreads) mx = fmaxf(mx, fabsf(x[i]));
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
    for (int64_t i = tid; i < k; i += kQThreads) q[i] = rintf(x[i] * c);
    if (tid == 0) step[0] = static_cast<float>(static_cast<double>(g) / 127.0);
}

// y[r] = (residual ? residual[r] : 0) + step * sum_s part[s][r], slices in order.
__global__ void __launch_bounds__(kEwThreads) k_w2a8_sum(const float *__restrict__ part, int64_t n, int ns,
                                                         const float *__restrict__ step,
                                                         const float *__restrict__ residual, float *__restrict__ y)
{
    const int64_t r = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x;
    if (r >= n) return;
    const float st = step[0];
    const float res = residual != nullptr ? residual[r] : 0.0f;
    float t = 0.0f;
    for (int s = 0; s < ns; ++s) t += part[static_cast<int64_t>(s) * n + r];
    y[r] = residual != nullptr ? fmaf(st, t, res) : st * t;
}

hipError_t launch_w2a8_quant(const float *x, int64_t k, float *q, float *step, hipStream_t s)
{
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
