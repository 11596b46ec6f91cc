// matvec_lut.hip -- batch-1 decode matvec with a per-slice lookup table.
//
// What is computed is the decode matvec of "A 27B model in 5.5 GB: Bonsai
// ternary on Ferrox, locally" ("What Ferrox does with it": each 28-byte
// block streamed once; "What Bonsai is": activations rotated first;
// "Speed, and where it goes": gate and up in one submission with SwiGLU
// and down following).  How it is computed differs from the pages' Metal
// design, which peels every trit with float arithmetic: on gfx950 that
// costs about 4 VALU operations per weight, more than the 1.5 operations
// per weight an HBM-bound matvec can afford at 8 TB/s.  Instead, since every
// row shares the same activation vector:
//
//   T[slot][b] = sum_n (digit_n(b) - 1) * xr[k(slot, n)]
//
// is tabulated once per workgroup for each byte position (slot) of a 2-block
// K-slice and each of the 256 byte values b.  A row's slice dot product is
// then sum_blocks scale * sum_slots T[slot][byte], one LDS lookup and one
// add per five weights.  Digits are decoded once per (slot, b) entry, not
// per weight.
//
// Layout on gfx950:
//   - K is cut into slices of 2 blocks (256 weights, 56 bytes per row); the
//     table of a slice is 56 slots x 256 fp32 in one 64 KB bank-interleaved
//     array, entry address = b << 8 | slot << 2, so one v_perm_b32
//     assembles the address from the data byte and a per-lane constant byte;
//     slots 26, 27 of each block (the scale bytes) hold zeros; at 64 KB, two
//     workgroups share a CU, so one's latency-bound phases (rotation, table
//     build, final reduction) overlap the other's lookups;
//   - weights are read in the tiled layout: the 32 rows x 2 blocks of a unit
//     are one contiguous 1792-byte tile, lane 2i + b holding block b of row
//     i, so a wave's loads are fully used 128-byte lines (a row-major matrix
//     would give each workgroup 56-byte pieces at the row pitch, which
//     measured at well under half the bandwidth);
//   - a workgroup (512 threads) owns one slice and a run of (matrix, 32-row
//     group) units of it; wave 0 rotates the slice's 1024-chunk of x in
//     registers, all threads build the table, then each of the 8 waves
//     processes exactly U units (U is a template parameter chosen per launch
//     so the grid fits two workgroups per CU), with all U units' weights
//     requested before the table is built; a lane reads its 28-byte block
//     with two wide loads and rotates its 7 dwords (and the byte order within
//     a dword) by a lane-dependent amount so the 32 lanes of a half-wave
//     (16 rows x 2 blocks) spread over LDS banks;
//   - a unit's 2 block partials (times their fp16 scales) are summed across
//     lanes with one xor-shuffle and written as split-K partials; a
//     per-group counter (atomicInc with wrap, so it is back to zero after
//     every launch) lets the last unit of a group sum the partials of all
//     slices in fixed order and apply the epilogue: store, + residual, or
//     (gate, up) -> RMS scale -> SwiGLU.  One launch, deterministic.
#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

constexpr int kLutBlocks = 2;                          // blocks per K-slice
constexpr int kLutSliceW = kLutBlocks * kBlockWeights;  // 256 weights
constexpr int kLutSlots = kLutBlocks * kBlockBytes;    // 56 byte slots
constexpr int kLutThreads = 512;
constexpr int kLutWaves = kLutThreads / kWave;         // 8
constexpr int kLutRows = 32;                           // rows per unit
constexpr int kLutTableBytes = 65536;                  // 256 byte values x 64 slot columns x fp32
static_assert(kLutRows == kTileRows && kLutBlocks == kTileBlocks, "a unit is one tile");
static_assert(kLutRows * kLutBlocks == kWave, "one block per lane");

// Per-lane dword rotation (rho) and byte rotation (sigma) for lanes 0..31
// (lanes 32..63 repeat them; lane 2i + b reads block b of row i): found by a
// search that minimises LDS bank collisions of the 32 slots a half-wave
// reads per lookup.
__constant__ uint8_t kLutRho[32] = {4, 6, 6, 1, 1, 5, 3, 2, 5, 3, 3, 3, 3, 6, 0, 5,
                                    1, 6, 3, 0, 2, 3, 1, 6, 6, 1, 6, 0, 4, 2, 0, 5};
__constant__ uint8_t kLutSig[32] = {0, 3, 1, 2, 1, 1, 1, 0, 0, 0, 3, 2, 0, 2, 1, 2,
                                    0, 1, 2, 1, 3, 1, 2, 0, 2, 3, 3, 0, 3, 3, 0, 3};

struct LutArgs {
    const uint8_t *w0, *w1;  // one or two tiled [n][k] matrices
    int64_t n, k;            // rows per matrix, K
    int nmat, nslices;
    int64_t groups;          // ceil(n / 32)
    int64_t units;           // nslices * nmat * groups
    int64_t units_per_wg;
    const float *x, *signs;
    float *part;             // [nslices][nmat][n]
    uint32_t *cnt;           // [groups], zero between launches
    // epilogue
    const float *residual;   // single matrix: y = residual + W xr
    float *y;
    float *g, *u, *h;        // two matrices: g, u (optional) and h = silu(a g) (a u)
    const float *x_rms;      // RMS scale source (nullptr: a = 1)
    int64_t d_rms;
    float rms_eps;
};

// T[slot][b] for b in [32 BQ, 32 BQ + 32): with v = floor(243 b / 256) the
// code of byte b and d_n its base-3 digits, T = ((d0-1) x0 + (d1-1) x1) +
// ((d2-1) x2 + (d3-1) x3 + (d4-1) x4); the digits are compile-time constants
// of the unrolled loop, so each entry is a few adds.
template <int BQ>
__device__ __forceinline__ void lut_build_range(float *tab, int slot, const float (&xv)[5])
{
    const uint32_t base = static_cast<uint32_t>(slot) << 2;  // slot < 64
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int b = 32 * BQ + i;
        const int v = (243 * b) >> 8;
        const float c0 = static_cast<float>(v / 81 - 1), c1 = static_cast<float>((v / 27) % 3 - 1);
        const float c2 = static_cast<float>((v / 9) % 3 - 1), c3 = static_cast<float>((v / 3) % 3 - 1);
        const float c4 = static_cast<float>(v % 3 - 1);
        const float t = (c0 * xv[0] + c1 * xv[1]) + (c2 * xv[2] + c3 * xv[3] + c4 * xv[4]);
        *reinterpret_cast<float *>(reinterpret_cast<char *>(tab) + (base | (static_cast<uint32_t>(b) << 8))) = t;
    }
}

// Split-K partials cross workgroups (and XCDs, whose L2s are not coherent
// for plain accesses): they are written and read with device-scope relaxed
// atomic accesses, which reach the coherence point themselves, instead of
// device-scope fences, which would write back and invalidate a whole L2.
__device__ __forceinline__ float lut_load_part(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void lut_store_part(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One unit = (slice s, matrix mat, 32-row group grp) = tile (grp, s) of
// matrix mat.  Row counts are below 2^20 (checked by the caller), so
// indices fit in int.
struct LutUnit {
    int mat, grp, r;
    bool live;
};

__device__ __forceinline__ LutUnit lut_unit(const LutArgs &a, int64_t un, int s, int64_t per_slice, int row_l,
                                           int blk_l, int nblk)
{
    LutUnit u;
    const int rem = static_cast<int>(un - static_cast<int64_t>(s) * per_slice);
    const int groups = static_cast<int>(a.groups);
    u.mat = rem >= groups ? 1 : 0;
    u.grp = rem - u.mat * groups;
    u.r = u.grp * kLutRows + row_l;
    u.live = (u.r < static_cast<int>(a.n)) && (blk_l < nblk);
    return u;
}

// A block's 7 dwords, read with two wide loads (16 + 12 bytes; blocks are
// only dword-aligned, which gfx950 global loads accept).  The lanes of a wave
// cover one 1792-byte tile.
typedef uint32_t lut_u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t lut_u32x3 __attribute__((ext_vector_type(3), aligned(4)));

__device__ __forceinline__ void lut_load(const LutArgs &a, const LutUnit &u, int s, int lane,
                                         uint32_t (&d)[kBlockDwords])
{
    // Unconditional loads (a branch around them would make the compiler wait
    // for each load before the next): padding rows and blocks of the tiled
    // layout exist (zero bytes) and their scale is zeroed by the caller.
    // Wave-uniform matrix base + 32-bit per-lane byte offset (tiled matrices
    // below 2 GiB, checked by the caller).
    const uint8_t *wm = u.mat ? a.w1 : a.w0;
    const uint32_t off = (static_cast<uint32_t>(u.grp) * static_cast<uint32_t>(a.nslices) +
                          static_cast<uint32_t>(s)) * kTileBytes + static_cast<uint32_t>(lane) * kBlockBytes;
    const lut_u32x4 lo = *reinterpret_cast<const lut_u32x4 *>(wm + off);
    const lut_u32x3 hi = *reinterpret_cast<const lut_u32x3 *>(wm + off + 16);
    d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
    d[4] = hi.x; d[5] = hi.y; d[6] = hi.z;
}

// d[j] <- d[(j + rho) mod 7]: a three-stage rotate by 1, 2 and 4.  The
// stages merge values with a lane mask (one v_bfi_b32 each); a select of
// array elements would become a dynamically indexed (private-memory) array.
__device__ __forceinline__ void lut_rotate(uint32_t (&d)[kBlockDwords], int rho)
{
#pragma unroll
    for (int sh = 1; sh <= 4; sh <<= 1) {
        const uint32_t m = (rho & sh) ? 0xffffffffu : 0u;
        uint32_t t[kBlockDwords];
#pragma unroll
        for (int j = 0; j < kBlockDwords; ++j) t[j] = (d[(j + sh) % kBlockDwords] & m) | (d[j] & ~m);
#pragma unroll
        for (int j = 0; j < kBlockDwords; ++j) d[j] = t[j];
    }
}

// Finish up to two completed row groups at once (one whole wave): lane =
// (group of the batch, row of the group); each lane sums its row's partials
// over all slices in slice order and applies the epilogue.  Every partial of
// a round of 16 slices is requested before any is summed.
__device__ void lut_finish(const LutArgs &a, const int (&grp)[2], int ngrp, int lane, float rms_a)
{
    constexpr int kPer = 16;
    const int gi = lane >> 5;
    const int64_t r_raw = gi < ngrp ? static_cast<int64_t>(grp[gi]) * kLutRows + (lane & (kLutRows - 1)) : a.n;
    const bool ok = r_raw < a.n;
    const int64_t r = ok ? r_raw : 0;  // clamped: every lane loads, no branch around the loads
    const int64_t stride = static_cast<int64_t>(a.nmat) * a.n;  // floats between slices
    const float *p0 = a.part + r;
    const float *p1 = a.part + (a.nmat == 2 ? a.n : 0) + r;
    float t0 = 0.0f, t1 = 0.0f;
    for (int q0 = 0; q0 < a.nslices; q0 += kPer) {
        float v0[kPer], v1[kPer];
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const int q = q0 + c < a.nslices ? q0 + c : a.nslices - 1;
            v0[c] = lut_load_part(p0 + q * stride);
            v1[c] = lut_load_part(p1 + q * stride);
        }
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            if (q0 + c < a.nslices) {
                t0 += v0[c];
                t1 += v1[c];
            }
        }
    }
    if (ok) {
        if (a.nmat == 1) {
            a.y[r] = a.residual ? a.residual[r] + t0 : t0;
        } else {
            const float gv = t0 * rms_a, uv = t1 * rms_a;
            if (a.g) a.g[r] = gv;
            if (a.u) a.u[r] = uv;
            if (a.h) a.h[r] = gv / (1.0f + expf(-gv)) * uv;
        }
    }
}

template <int U>
__global__ void __launch_bounds__(kLutThreads, 2) k_matvec_lut(LutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float *tab = reinterpret_cast<float *>(lds);                 // 64 KB table
    float *xs = reinterpret_cast<float *>(lds + kLutTableBytes);  // 256 floats
    float *red = xs + kLutSliceW;                               // 16 floats

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int s = blockIdx.y;                                      // the slice
    const int64_t per_slice = static_cast<int64_t>(a.nmat) * a.groups;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kLutWaves + wave) * U;  // this wave's first unit
    const int64_t k0 = static_cast<int64_t>(s) * kLutSliceW;
    const int kw = static_cast<int>(a.k - k0 < kLutSliceW ? a.k - k0 : kLutSliceW);
    const int nblk = kw / kBlockWeights;
    const int row_l = lane >> 1;  // row of the unit (tile) this lane reads
    const int blk_l = lane & 1;   // block of the slice this lane reads
    const int rho = kLutRho[lane & 31], sig = kLutSig[lane & 31];

    // ---- this wave's U units of weights, requested before anything else
    uint32_t dat[U][kBlockDwords];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int64_t un = first + i < per_slice ? first + i : per_slice - 1;  // clamped: no branch
        lut_load(a, lut_unit(a, un + static_cast<int64_t>(s) * per_slice, s, per_slice, row_l, blk_l, nblk),
                 s, lane, dat[i]);
    }

    // ---- RMS scale of the block input (gate/up epilogue only)
    float rms_a = 1.0f;
    if (a.x_rms != nullptr) {
        float sq = 0.0f;
        for (int64_t i = tid; i < a.d_rms; i += kLutThreads) sq = fmaf(a.x_rms[i], a.x_rms[i], sq);
#pragma unroll
        for (int h = kWave / 2; h > 0; h >>= 1) sq += __shfl_xor(sq, h, kWave);
        if (lane == 0) red[wave] = sq;
    }
    // ---- x for this slice (rotated when signs are given: k % 1024 == 0)
    if (a.signs != nullptr) {
        if (wave == 0) {
            const int64_t c0 = (k0 / kHadamard) * kHadamard;
            const int part = static_cast<int>(k0 - c0);  // 0, 256, 512 or 768
            float v[kRotPerLane];
#pragma unroll
            for (int j = 0; j < kRotPerLane; ++j) v[j] = a.x[c0 + lane + kWave * j] * a.signs[lane + kWave * j];
            fwht1024_wave(v);
#pragma unroll
            for (int j = 0; j < kRotPerLane; ++j) {
                const int e = lane + kWave * j - part;
                if (e >= 0 && e < kLutSliceW) xs[e] = v[j] * (1.0f / 32.0f);
            }
        }
    } else {
        for (int i = tid; i < kLutSliceW; i += kLutThreads) xs[i] = i < kw ? a.x[k0 + i] : 0.0f;
    }
    __syncthreads();
    if (a.x_rms != nullptr) {
        float t = 0.0f;
        for (int w = 0; w < kLutWaves; ++w) t += red[w];
        rms_a = 1.0f / sqrtf(t / static_cast<float>(a.d_rms) + a.rms_eps);
    }
    // ---- table: thread = (slot, 32-value range of the byte)
    {
        const int bq = tid >> 6;  // 0..7
        const int slot = tid & 63;
        if (slot < kLutSlots) {
            const int blk = slot / kBlockBytes, i = slot % kBlockBytes;
            float xv[5];
#pragma unroll
            for (int n = 0; n < 5; ++n) {
                const int j = kTritsPerByte * i + n;  // weight index in the block
                xv[n] = (blk < nblk && i < kTritBytes && j < kBlockWeights) ? xs[blk * kBlockWeights + j] : 0.0f;
            }
            switch (bq) {
                case 0: lut_build_range<0>(tab, slot, xv); break;
                case 1: lut_build_range<1>(tab, slot, xv); break;
                case 2: lut_build_range<2>(tab, slot, xv); break;
                case 3: lut_build_range<3>(tab, slot, xv); break;
                case 4: lut_build_range<4>(tab, slot, xv); break;
                case 5: lut_build_range<5>(tab, slot, xv); break;
                case 6: lut_build_range<6>(tab, slot, xv); break;
                default: lut_build_range<7>(tab, slot, xv); break;
            }
        }
    }
    __syncthreads();

    // ---- per-lane lookup constants.  Address of the lookup for byte c of
    // the lane's j-th dword: byte << 8 | slot << 2; the four slot bytes of a
    // dword are packed in one register (byte c) and v_perm_b32 inserts the
    // data byte (selector: byte 0 <- P byte c, byte 1 <- data byte e, 0, 0).
    uint32_t P[kBlockDwords];
    uint32_t S[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t e = static_cast<uint32_t>((c + sig) & 3);
        S[c] = 0x0C0C0000u | (e << 8) | static_cast<uint32_t>(4 + c);
    }
#pragma unroll
    for (int j = 0; j < kBlockDwords; ++j) {
        const int q = (j + rho) % kBlockDwords;
        uint32_t packed = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int slot = kBlockBytes * blk_l + 4 * q + ((c + sig) & 3);
            packed |= (static_cast<uint32_t>(slot) << 2) << (8 * c);
        }
        P[j] = packed;
    }

    // ---- lookups, scale, 2-lane reduction, partial store
    typedef __attribute__((address_space(3))) const float lds_f32;
    int my_grp = 0;  // lane i records the group of unit i
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const bool unit_ok = first + i < per_slice;  // wave-uniform
        const int64_t un = unit_ok ? first + i : per_slice - 1;
        const LutUnit u = lut_unit(a, un + static_cast<int64_t>(s) * per_slice, s, per_slice, row_l, blk_l, nblk);
        const float scale = (u.live && unit_ok) ? half_bits_to_float(dat[i][kBlockDwords - 1] >> 16) : 0.0f;
        lut_rotate(dat[i], rho);
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int j = 0; j < kBlockDwords; ++j) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t addr = __builtin_amdgcn_perm(P[j], dat[i][j], S[c]);
                const float t = *reinterpret_cast<lds_f32 *>(static_cast<uintptr_t>(addr));
                if ((c & 1) == 0) acc0 += t; else acc1 += t;
            }
        }
        float p = (acc0 + acc1) * scale;
        p += __shfl_xor(p, 1, kWave);
        if (unit_ok && blk_l == 0 && u.r < a.n)
            lut_store_part(a.part + (static_cast<int64_t>(s) * a.nmat + u.mat) * a.n + u.r, p);
        if (lane == i) my_grp = u.grp;
    }

    // ---- arrivals: all partial stores complete at the coherence point
    // (s_waitcnt vmcnt(0); gfx9 encoding, expcnt/lgkmcnt not waited), then
    // one atomic per lane counts unit `lane`; the last arrival of a row group
    // sums that group's partials over all slices and finishes it.
    const int nu = first < per_slice ? static_cast<int>(per_slice - first < U ? per_slice - first : U) : 0;
    if (nu > 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        const uint32_t target = static_cast<uint32_t>(a.nslices * a.nmat);
        uint32_t old = 0;
        if (lane < nu) old = atomicInc(&a.cnt[my_grp], target - 1u);
        uint64_t last = __ballot(lane < nu && old == target - 1u);
        while (last) {
            int grp2[2];
            int ng = 0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                grp2[q] = 0;
                if (last) {
                    const int i = __builtin_ctzll(last);
                    last &= last - 1;
                    grp2[q] = __shfl(my_grp, i, kWave);
                    ng = q + 1;
                }
            }
            lut_finish(a, grp2, ng, lane, rms_a);
        }
    }
}

static int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

size_t lut_part_floats(int64_t n, int nmat, int64_t k)
{
    const int64_t nslices = (k + kLutSliceW - 1) / kLutSliceW;
    return static_cast<size_t>(nslices * nmat * n);
}

size_t lut_counter_words(int64_t n) { return static_cast<size_t>((n + kLutRows - 1) / kLutRows); }

template <int U>
static hipError_t lut_launch(const LutArgs &a, int64_t chunks, hipStream_t st)
{
    static bool attr_done = false;
    const size_t lds = kLutTableBytes + (kLutSliceW + kLutWaves) * sizeof(float);
    if (!attr_done) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_matvec_lut<U>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    hipLaunchKernelGGL(k_matvec_lut<U>, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(a.nslices)),
                       dim3(kLutThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_matvec_lut(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k,
                             const float *x, const float *signs, float *part, uint32_t *cnt,
                             const float *residual, float *y, float *g, float *u, float *h,
                             const float *x_rms, int64_t d_rms, float rms_eps, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    LutArgs a{};
    a.w0 = w0;
    a.w1 = w1;
    a.n = n;
    a.k = k;
    a.nmat = nmat;
    a.nslices = static_cast<int>((k + kLutSliceW - 1) / kLutSliceW);
    a.groups = (n + kLutRows - 1) / kLutRows;
    a.units = static_cast<int64_t>(a.nslices) * nmat * a.groups;
    a.x = x;
    a.signs = signs;
    a.part = part;
    a.cnt = cnt;
    a.residual = residual;
    a.y = y;
    a.g = g;
    a.u = u;
    a.h = h;
    a.x_rms = x_rms;
    a.d_rms = d_rms;
    a.rms_eps = rms_eps;
    // units per wave: the smallest U whose grid (slices x chunks of 8U units)
    // fits two workgroups per CU in one round, else the largest U
    const int64_t per_slice = static_cast<int64_t>(nmat) * a.groups;
    const int cus = device_cus();
    static const int kUs[] = {1, 2, 3, 4, 6, 8};
    int U = 8;
    for (int cand : kUs) {
        const int64_t chunks = (per_slice + kLutWaves * cand - 1) / (kLutWaves * cand);
        if (chunks * a.nslices <= 2 * static_cast<int64_t>(cus)) {
            U = cand;
            break;
        }
    }
    const int64_t chunks = (per_slice + kLutWaves * U - 1) / (kLutWaves * U);
    a.units_per_wg = static_cast<int64_t>(kLutWaves) * U;
    switch (U) {
        case 1: return lut_launch<1>(a, chunks, s);
        case 2: return lut_launch<2>(a, chunks, s);
        case 3: return lut_launch<3>(a, chunks, s);
        case 4: return lut_launch<4>(a, chunks, s);
        case 6: return lut_launch<6>(a, chunks, s);
        default: return lut_launch<8>(a, chunks, s);
    }
}

}  // namespace ptq1
