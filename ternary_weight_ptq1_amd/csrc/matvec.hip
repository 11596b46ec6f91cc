// matvec.hip -- element-wise SwiGLU, h = silu(g) * u with silu(z) =
// z / (1 + e^-z) ("A 27B model in 5.5 GB: Bonsai ternary on Ferrox,
// locally", section "Speed, and where it goes": gate, SwiGLU, down).  The
// decode path fuses it into the gate/up sum (matvec_lut.hip) and the prefill
// path into the activation prep (gemm.hip); this kernel serves
// ptq1_swiglu.
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

__global__ void __launch_bounds__(kEwThreads) k_swiglu(const float *g, const float *u, float *h, int64_t len)
{
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x; i < len;
         i += static_cast<int64_t>(gridDim.x) * kEwThreads)
        h[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
}

hipError_t launch_swiglu(const float *g, const float *u, float *h, int64_t len, hipStream_t s)
{
    if (len == 0) return hipSuccess;
    int64_t blocks = (len + kEwThreads - 1) / kEwThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_swiglu, dim3(static_cast<unsigned>(blocks)), dim3(kEwThreads), 0, s, g, u, h, len);
    return hipGetLastError();
}

}  // namespace ptq1
