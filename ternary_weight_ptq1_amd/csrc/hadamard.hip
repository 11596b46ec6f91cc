// hadamard.hip -- activation rotation and embedding-row unrotation.
//
// "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally", section "What
// Bonsai is": a 1024-wide Walsh-Hadamard butterfly with a sign pattern,
// applied to activations before every folded matmul and undone on embedding
// rows after lookup.  R = (1/32) H D_s per 1024-chunk; R^T = (1/32) D_s H.
//
// One wavefront per chunk: the butterfly runs in registers and cross-lane
// shuffles (no LDS, no barriers); loads and stores are fully coalesced
// (lane l touches elements l + 64 j).
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

// x and y may be the same buffer: a wave reads its whole chunk before writing.
__global__ void __launch_bounds__(kRotThreads) k_rotate(const float *x, float *y, int64_t nchunks,
                                                        const float *__restrict__ signs)
{
    const int64_t c = blockIdx.x;
    if (c >= nchunks) return;
    const int lane = threadIdx.x;
    const float *src = x + c * kHadamard;
    float v[kRotPerLane];
#pragma unroll
    for (int j = 0; j < kRotPerLane; ++j) v[j] = src[lane + kWave * j] * signs[lane + kWave * j];
    fwht1024_wave(v);
    float *dst = y + c * kHadamard;
#pragma unroll
    for (int j = 0; j < kRotPerLane; ++j) dst[lane + kWave * j] = v[j] * (1.0f / 32.0f);
}

__global__ void __launch_bounds__(kRotThreads) k_unrotate_rows(const float *__restrict__ table,
                                                               int64_t n_table, int64_t d,
                                                               const int32_t *__restrict__ ids,
                                                               const float *__restrict__ signs,
                                                               float *__restrict__ out)
{
    const int64_t cpr = d / kHadamard;  // chunks per row
    const int64_t row = blockIdx.x / cpr;
    const int64_t ch = blockIdx.x - row * cpr;
    const int lane = threadIdx.x;
    // the signs are requested before the id (the row's address waits for
    // the id; loaded after the rotation they cost a third round trip)
    float sg[kRotPerLane];
#pragma unroll
    for (int j = 0; j < kRotPerLane; ++j) sg[j] = signs[lane + kWave * j];
    const int64_t id = ids ? static_cast<int64_t>(ids[row]) : row;
    float *dst = out + row * d + ch * kHadamard;
    if (id < 0 || id >= n_table) {  // out-of-range id: a NaN row, no access
#pragma unroll
        for (int j = 0; j < kRotPerLane; ++j) dst[lane + kWave * j] = __builtin_nanf("");
        return;
    }
    const float *src = table + id * d + ch * kHadamard;
    float v[kRotPerLane];
#pragma unroll
    for (int j = 0; j < kRotPerLane; ++j) v[j] = src[lane + kWave * j];
    fwht1024_wave(v);
#pragma unroll
    for (int j = 0; j < kRotPerLane; ++j)
        dst[lane + kWave * j] = v[j] * (1.0f / 32.0f) * sg[j];
}

hipError_t launch_rotate(const float *x, float *y, int64_t m, int64_t k, const float *signs,
                         hipStream_t s)
{
    const int64_t nchunks = m * (k / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rotate, dim3(static_cast<unsigned>(nchunks)), dim3(kRotThreads), 0, s, x,
                       y, nchunks, signs);
    return hipGetLastError();
}

hipError_t launch_unrotate_rows(const float *table, int64_t n_table, int64_t d, const int32_t *ids,
                                int64_t n_rows, const float *signs, float *out, hipStream_t s)
{
    const int64_t nchunks = n_rows * (d / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_unrotate_rows, dim3(static_cast<unsigned>(nchunks)), dim3(kRotThreads), 0,
                       s, table, n_table, d, ids, signs, out);
    return hipGetLastError();
}

}  // namespace ptq1
