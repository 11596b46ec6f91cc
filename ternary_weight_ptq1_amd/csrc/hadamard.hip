// hadamard.hip -- activation rotation and embedding-row unrotation.
//
// "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally", section "What
// Bonsai is": a 1024-wide Walsh-Hadamard butterfly with a sign pattern,
// applied to activations before every folded matmul and undone on embedding
// rows after lookup.  R = (1/32) H D_s per 1024-chunk; R^T = (1/32) D_s H.
//
// Four waves per chunk: each transforms a 256-wide quarter with the
// butterfly in registers and cross-lane shuffles, and the quarters meet in
// one exchange through LDS (H_1024 = H_4 (x) H_256).  Loads and stores are
// 16 bytes per lane and coalesced.  A decode step rotates or unrotates a
// handful of chunks, so the length of one chunk's dependent chain is what
// counts: a quarter of the one-wave transform.
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

// y = R x chunk by chunk, R = (1/32) H_1024 D_s, four waves per chunk as in
// the unrotation below (wave w transforms quarter w, then forms output
// quarter w).  x and y may be the same buffer: every read of a chunk
// happens before the barrier, every write after it.
constexpr int kQuarterThreads = 4 * kWave;

__global__ void __launch_bounds__(kQuarterThreads) k_rotate(const float *x, float *y, int64_t nchunks,
                                                            const float *__restrict__ signs)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ f32x4 qt[kQuarterThreads];  // H_256 of each quarter, 4 KB
    const int64_t c = blockIdx.x;
    if (c >= nchunks) return;  // workgroup-uniform
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int e = (kHadamard / 4) * w + 4 * lane;
    const f32x4 xv = *reinterpret_cast<const f32x4 *>(x + c * kHadamard + e);
    const f32x4 sg = *reinterpret_cast<const f32x4 *>(signs + e);
    float v[4] = {xv[0] * sg[0], xv[1] * sg[1], xv[2] * sg[2], xv[3] * sg[3]};
    fwht256_wave(v);
    qt[tid] = f32x4{v[0], v[1], v[2], v[3]};
    __syncthreads();
    const f32x4 q0 = qt[lane], q1 = qt[kWave + lane], q2 = qt[2 * kWave + lane], q3 = qt[3 * kWave + lane];
    const float s1 = (w & 1) ? -1.0f : 1.0f, s2 = (w & 2) ? -1.0f : 1.0f;  // row w of H_4
    const f32x4 t = (q0 + s1 * q1) + s2 * (q2 + s1 * q3);
    *reinterpret_cast<f32x4 *>(y + c * kHadamard + e) = t * (1.0f / 32.0f);
}

// out[row] = R^T table[ids[row]], chunk by chunk; an out-of-range id gives a
// row of NaNs.  Four waves per chunk: wave w transforms quarter w (elements
// 256 w + 4 lane + k, one 16-byte load per array) with the 256-point
// butterfly in registers, the four quarter transforms meet in LDS, and wave
// w forms output quarter w = sum_c (-1)^popcount(w & c) H_256 quarter c
// (H_1024 = H_4 (x) H_256, the top two index bits being the H_4 factor).
// A chunk's dependent chain is thus a quarter of the one-wave transform.
__global__ void __launch_bounds__(kQuarterThreads) k_unrotate_rows(const float *__restrict__ table,
                                                                 int64_t n_table, int64_t d,
                                                                 const int32_t *__restrict__ ids,
                                                                 const float *__restrict__ signs,
                                                                 float *__restrict__ out)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ f32x4 qt[kQuarterThreads];  // H_256 of each quarter, 4 KB
    const int64_t cpr = d / kHadamard;  // chunks per row
    const int64_t row = blockIdx.x / cpr;
    const int64_t ch = blockIdx.x - row * cpr;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;  // quarter
    const int e = (kHadamard / 4) * w + 4 * lane;  // this thread's four elements of the chunk
    // the signs are requested before the id (the row's address waits for
    // the id; loaded after the rotation they cost a third round trip)
    const f32x4 sg = *reinterpret_cast<const f32x4 *>(signs + e);
    const int64_t id = ids ? static_cast<int64_t>(ids[row]) : row;
    float *dst = out + row * d + ch * kHadamard;
    if (id < 0 || id >= n_table) {  // out-of-range id (the same for the whole workgroup): NaNs, no access
        const float nan = __builtin_nanf("");
        *reinterpret_cast<f32x4 *>(dst + e) = f32x4{nan, nan, nan, nan};
        return;
    }
    const f32x4 x = *reinterpret_cast<const f32x4 *>(table + id * d + ch * kHadamard + e);
    float v[4] = {x[0], x[1], x[2], x[3]};
    fwht256_wave(v);
    qt[tid] = f32x4{v[0], v[1], v[2], v[3]};
    __syncthreads();
    const f32x4 q0 = qt[lane], q1 = qt[kWave + lane], q2 = qt[2 * kWave + lane], q3 = qt[3 * kWave + lane];
    const float s1 = (w & 1) ? -1.0f : 1.0f, s2 = (w & 2) ? -1.0f : 1.0f;  // row w of H_4
    const f32x4 t = (q0 + s1 * q1) + s2 * (q2 + s1 * q3);
    *reinterpret_cast<f32x4 *>(dst + e) = t * (1.0f / 32.0f) * sg;
}

hipError_t launch_rotate(const float *x, float *y, int64_t m, int64_t k, const float *signs,
                         hipStream_t s)
{
    const int64_t nchunks = m * (k / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rotate, dim3(static_cast<unsigned>(nchunks)), dim3(kQuarterThreads), 0, s, x,
                       y, nchunks, signs);
    return hipGetLastError();
}

hipError_t launch_unrotate_rows(const float *table, int64_t n_table, int64_t d, const int32_t *ids,
                                int64_t n_rows, const float *signs, float *out, hipStream_t s)
{
    const int64_t nchunks = n_rows * (d / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_unrotate_rows, dim3(static_cast<unsigned>(nchunks)), dim3(kQuarterThreads), 0,
                       s, table, n_table, d, ids, signs, out);
    return hipGetLastError();
}

}  // namespace ptq1
