// w2a8.hip -- the row steps of the 8-bit-activation prefill GEMM ("Why I Am
// Building Another Inference Engine", Level 5: integer kernels pair ternary
// weights with int8 activations, the numerics BitNet b1.58 was trained with;
// Level 4: a BitNet layer rounds its activations to int8 ahead of its ternary
// matmuls).  The decode matvec's quantiser runs inside the lookup kernel
// (matvec_lut.hip).
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

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

}  // namespace ptq1
