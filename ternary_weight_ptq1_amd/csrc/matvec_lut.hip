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
//   T[slot][b] = sum_n (digit_n(b) - 1) * q[k(slot, n)]
//
// is tabulated once per workgroup for each byte position (slot) of a 2-block
// K-slice and each of the 256 byte values b, where q = rint(xr 2^e) holds the
// slice's rotated activations in 32-bit fixed point (one power of two 2^e
// per slice, |q| < 2^23).  A row's slice dot product is then
// 2^-e sum_blocks scale * sum_slots T[slot][byte]: one LDS lookup per five
// weights and one integer add (v_add3_u32) per two lookups, the block sums
// exact in int32.  Digits are decoded once per (slot, b) entry, not per
// weight.  The one rounding beyond fp32 is that of xr to q, at most 2^-24
// of the slice's max|xr| per element.
//
// Layout on gfx950:
//   - K is cut into slices of 2 blocks (256 weights, 56 bytes per row); the
//     table of a slice has 64 columns (32 per block: byte positions 0..25
//     are the trit bytes, 26..31 columns of zeros) x 256 byte values, int32,
//     in one 64 KB array, entry address = b << 8 | column << 2, so an
//     entry's LDS bank is its column mod 32 and one v_perm_b32 assembles the
//     address from the data byte and a per-lane constant byte; at 64 KB, two
//     workgroups share a CU, and the prologue (x, rotation, table build)
//     runs at raised wave priority, so a workgroup that starts late on a CU
//     builds its table ahead of the other one's lookups;
//   - weights are read in the tiled layout: the 32 rows x 2 blocks of a unit
//     are one contiguous 1792-byte tile, lane 2i + b holding block b of row
//     i, so a wave's loads are fully used 128-byte lines (a row-major matrix
//     would give each workgroup 56-byte pieces at the row pitch, which
//     measured at well under half the bandwidth); tiles are K-slice-major,
//     so the units a workgroup walks (consecutive row bands of one slice)
//     are one contiguous run of memory, and so are its neighbours';
//   - a workgroup (512 threads) owns one slice and a run of (matrix, 32-row
//     group) units of it; wave 0 rotates x for the slice in registers (its
//     loads requested before any weights: vector-memory loads return in
//     order; only the slice's 256 outputs of the 1024-chunk's transform are
//     formed, see lut_fwht256), all threads build the table, and each of the 8 waves
//     processes U units (U is a template parameter chosen per launch so the
//     grid fits two workgroups per CU) with kLutDepth units of weights in
//     flight (one requested before x arrives, after wave 0's x requests have
//     gone out, so that x is not queued behind a chip-wide burst of weight
//     requests); a lane reads its 28-byte block
//     with two wide loads and rotates its 8 dwords (the 7 of the block and a
//     zero) and the byte order within a dword by lane-dependent amounts
//     (lut_rho, lut_sig), which with block 1's columns shifted by 16 banks
//     makes the 32 lanes of every half-wave lookup read 32 different banks:
//     no LDS bank conflicts;
//   - a unit's 2 block partials (times their fp16 scales) are summed across
//     neighbouring lanes (one DPP move) and stored as split-K partials
//     part[slice][matrix][row]; a second kernel sums each row's partials in
//     slice order and applies the epilogue (+ residual, or RMS scale and
//     SwiGLU).  The kernel boundary makes the partials visible across XCDs
//     at once; finishing inside the matvec kernel instead (arrival counters
//     and device-scope loads that bypass the L2) measured slower, its
//     round trips to memory sitting at the end of the critical path.
#include <hip/hip_ext.h>

#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

constexpr int kLutBlocks = 2;                          // blocks per K-slice
constexpr int kLutSliceW = kLutBlocks * kBlockWeights;  // 256 weights
#ifndef PTQ1_LUT_THREADS
#define PTQ1_LUT_THREADS 512
#endif
constexpr int kLutThreads = PTQ1_LUT_THREADS;          // one workgroup: kLutWgPerCu per CU
constexpr int kLutWaves = kLutThreads / kWave;
constexpr int kLutWgPerCu = 1024 / kLutThreads;        // 64 KB of LDS each
constexpr int kLutBuildRanges = kLutThreads / kWave;   // table build: threads = (slot, byte range)
constexpr int kLutBuildPer = 256 / kLutBuildRanges;    // byte values per thread
constexpr int kLutRows = 32;                           // rows per unit
constexpr int kLutTableBytes = 65536;                  // 256 byte values x 64 slot columns x fp32
#ifndef PTQ1_LUT_EARLY
#define PTQ1_LUT_EARLY 1
#endif
#ifndef PTQ1_LUT_DEPTH
#define PTQ1_LUT_DEPTH 3
#endif
constexpr int kLutEarly = PTQ1_LUT_EARLY;              // units per wave requested before x arrives
constexpr int kLutDepth = PTQ1_LUT_DEPTH;              // units of weights in flight per wave
static_assert(kLutEarly >= 1 && kLutEarly <= kLutDepth, "at least one unit before x, at most the depth");
typedef uint32_t lut_u32x3 __attribute__((ext_vector_type(3), aligned(4)));
static_assert(kLutRows == kTileRows && kLutBlocks == kTileBlocks, "a unit is one tile");
static_assert(kLutRows * kLutBlocks == kWave, "one block per lane");

// Table columns: byte position p (0..31) of block b of the slice is column
// 32 b + (p + 16 b) mod 32.  Positions 0..25 are the trit bytes; 26, 27 (the
// scale) and 28..31 (past the block) are columns of zeros.  Entry (column,
// byte value v) sits at byte v * 256 + column * 4, so its LDS bank (32 banks
// of 4 bytes) is p for block 0 and p + 16 mod 32 for block 1.
constexpr int kLutColsPerBlock = 32;
constexpr int kLutDwords = kLutColsPerBlock / 4;  // 8 dword positions per block, 7 of them in memory
static_assert(kLutBlocks * kLutColsPerBlock * 256 * 4 == 65536, "the table fills 64 KB");

// Lane 2i + b (row i, block b of a tile) holds in register r dword
// q = (r + rho) mod 8 of its block and reads byte (c + sig) mod 4 of it at
// step c, with rho = (i / 4) mod 4 and sig = i mod 4: in a half-wave (rows
// 0..15 or 16..31, which the LDS serves in one pass) the 16 lanes of a block
// hold the 16 pairs (rho, sig), so at step (r, c) block 0 reads the 16 banks
// of dword positions r .. r + 3 (mod 8) and block 1, its columns shifted by
// 16 banks, the other 16: no two lanes of a half-wave share a bank.  The
// shift puts half of the spread into the table's layout, so the data is
// rotated by 0..3 dwords (two rounds of selects) instead of 0..7.
__device__ __forceinline__ int lut_rho(int lane) { return (lane >> 3) & 3; }
__device__ __forceinline__ int lut_sig(int lane) { return (lane >> 1) & 3; }

struct LutArgs {
    const uint8_t *w0, *w1;  // one or two tiled [n][k] matrices
    int64_t n, k;            // rows per matrix, K
    int nmat, nslices;
    int64_t groups;          // ceil(n / 32)
    int per_wg;              // units of a slice per workgroup (the last workgroup of a slice may get fewer)
    const float *x, *signs;  // x [k], rotated here when signs != nullptr
    const float *gain;       // [k] or nullptr: x is used as gain * x (a norm's per-channel weight)
    float *part;             // [nslices][nmat][n]
};

// ---------------------------------------------------------------------------
// Rotation of one slice's 256 activations.  In natural order H_1024 =
// H_4 (x) H_256 (the top two index bits are the H_4 factor), so outputs
// 256 p .. 256 p + 255 of a 1024-chunk are the 256-point transform of
// z_d = sum_c (-1)^popcount(p & c) s[256 c + d] x[256 c + d]: one wave, four
// values per lane (six bits of d in the lane index, two in the register
// index), butterflies across lanes by DPP and the gfx950 lane-swap
// instructions (no LDS traffic), the two in-lane stages in registers.  A butterfly leaves x_i + x_(i^h) at the lane whose bit h is 0
// and x_(i^h) - x_i at the other: partner + sgn * own, sgn = +-1.
// ---------------------------------------------------------------------------
template <int kRowShl, int kRowShr>
__device__ __forceinline__ float lut_dpp(float v, bool upper)
{
    const int iv = __builtin_bit_cast(int, v);
    const int lo = __builtin_amdgcn_update_dpp(iv, iv, kRowShl, 0xF, 0xF, false);  // lane + h
    const int hi = __builtin_amdgcn_update_dpp(iv, iv, kRowShr, 0xF, 0xF, false);  // lane - h
    return __builtin_bit_cast(float, upper ? hi : lo);
}

__device__ __forceinline__ void lut_fwht256(float (&v)[4], int lane)
{
    // lane bits 0, 1: quad permutations
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int iv = __builtin_bit_cast(int, v[k]);
        const float p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0xB1, 0xF, 0xF, false));
        v[k] = fmaf((lane & 1) ? -1.0f : 1.0f, v[k], p);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int iv = __builtin_bit_cast(int, v[k]);
        const float p = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0x4E, 0xF, 0xF, false));
        v[k] = fmaf((lane & 2) ? -1.0f : 1.0f, v[k], p);
    }
    // lane bits 2, 3: row shifts by 4 and 8 (within 16-lane rows)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = fmaf((lane & 4) ? -1.0f : 1.0f, v[k], lut_dpp<0x104, 0x114>(v[k], lane & 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = fmaf((lane & 8) ? -1.0f : 1.0f, v[k], lut_dpp<0x108, 0x118>(v[k], lane & 8));
    // lane bits 4, 5: swaps of 16-lane rows and of 32-lane halves between
    // two copies of the value; result [0] holds the own value in the lower
    // part and the partner's above, result [1] the partner's below and the
    // own value above.  (The elements are copied to scalars before the bit
    // cast: a bit cast of an element of the returned pair reads element 0.)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v[k]);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        v[k] = fmaf((lane & 16) ? -1.0f : 1.0f, __builtin_bit_cast(float, r1), __builtin_bit_cast(float, r0));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v[k]);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        v[k] = fmaf((lane & 32) ? -1.0f : 1.0f, __builtin_bit_cast(float, r1), __builtin_bit_cast(float, r0));
    }
    // value bits 0, 1 (d bits 6, 7): in registers
    float t0 = v[0] + v[1], t1 = v[0] - v[1], t2 = v[2] + v[3], t3 = v[2] - v[3];
    v[0] = t0 + t2;
    v[1] = t1 + t3;
    v[2] = t0 - t2;
    v[3] = t1 - t3;
}

// ---------------------------------------------------------------------------
// x of one 256-wide K-slice, loaded by one wave before anything else: with
// signs, the four quarters of the 1024-chunk holding the slice (lane l holds
// elements 256 c + 4 l .. 256 c + 4 l + 3 of quarter c, one 16-byte load per
// quarter and array); without, the slice itself (elements 4 l .. 4 l + 3,
// clamped into the slice when it is a 128-wide tail).  The FWHT above does
// not depend on which index bits sit in lanes and which in registers, so
// with d = 4 l + k the slice's outputs come back as xs[4 l + k].
// ---------------------------------------------------------------------------
typedef float lut_f32x4 __attribute__((ext_vector_type(4)));

struct SliceX {
    lut_f32x4 x[4], s[4], g[4];
};

__device__ __forceinline__ void slice_x_load(const float *x, const float *signs, const float *gain, int64_t k0, int kw,
                                             int lane, SliceX &v)
{
    if (signs != nullptr) {
        const int64_t c0 = (k0 / kHadamard) * kHadamard;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v.x[c] = *reinterpret_cast<const lut_f32x4 *>(x + c0 + kLutSliceW * c + 4 * lane);
            v.s[c] = *reinterpret_cast<const lut_f32x4 *>(signs + kLutSliceW * c + 4 * lane);
        }
        if (gain != nullptr) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v.g[c] = *reinterpret_cast<const lut_f32x4 *>(gain + c0 + kLutSliceW * c + 4 * lane);
        }
    } else {
        const int e = 4 * lane < kw ? 4 * lane : kw - 4;  // clamped; zeroed when stored
        v.x[0] = *reinterpret_cast<const lut_f32x4 *>(x + k0 + e);
        if (gain != nullptr) v.g[0] = *reinterpret_cast<const lut_f32x4 *>(gain + k0 + e);
    }
}

// This lane's four values of the slice of R (gain * x) (or of gain * x when
// signs == nullptr), elements 4 lane .. 4 lane + 3.
__device__ __forceinline__ lut_f32x4 slice_x_values(const SliceX &v, bool rotate, bool gained, int64_t k0, int kw,
                                                    int lane)
{
    lut_f32x4 out;
    if (rotate) {
        const int part = static_cast<int>((k0 % kHadamard) / kLutSliceW);  // 0..3: this slice's quarter
        const float sa = (part & 1) ? -1.0f : 1.0f, sb = (part & 2) ? -1.0f : 1.0f;
        float z[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float t[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = (gained ? v.x[c][k] * v.g[c][k] : v.x[c][k]) * v.s[c][k];
            z[k] = fmaf(sa, t[1], t[0]) + sb * fmaf(sa, t[3], t[2]);  // row `part` of H_4
        }
        lut_fwht256(z, lane);
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = z[k] * (1.0f / 32.0f);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            out[k] = 4 * lane + k < kw ? (gained ? v.x[0][k] * v.g[0][k] : v.x[0][k]) : 0.0f;
    }
    return out;
}

// xs[0..256) = the slice (see slice_x_values), fp32
__device__ __forceinline__ void slice_x_store(const SliceX &v, bool rotate, bool gained, int64_t k0, int kw, int lane,
                                              float *xs)
{
    *reinterpret_cast<lut_f32x4 *>(xs + 4 * lane) = slice_x_values(v, rotate, gained, k0, kw, lane);
}

// The slice in 32-bit fixed point, one power of two per slice: with
// max |x| = f 2^E (f in [0.5, 1); E = 0 for an all-zero slice) and e = 23 - E,
// q = rint(x 2^e) is exact scaling followed by one rounding to the nearest
// integer, |q| <= 2^23, and any sum of a block's 26 table entries (each a sum
// of five +-q) stays below 130 * 2^23 < 2^31.  xs[0..256) receives q as
// int32, ex[0] the exponent e and ex[1] the slice's factor: 1, or a NaN when
// the slice holds a NaN or an infinity (whose products a fixed-point sum
// cannot carry; every output the slice feeds then becomes a NaN).
__device__ __forceinline__ void slice_x_store_fixed(const lut_f32x4 &v, int lane, float *xs, float *ex)
{
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    const bool bad = !(__builtin_isfinite(v[0]) && __builtin_isfinite(v[1]) && __builtin_isfinite(v[2]) &&
                       __builtin_isfinite(v[3]));
    const bool any_bad = __ballot(bad) != 0;  // wave-uniform
    m = wave_max(m);
    int E = 0;
    (void)frexpf(any_bad ? 0.0f : m, &E);
    const int e = 23 - E;
    int32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = any_bad ? 0 : static_cast<int32_t>(rintf(ldexpf(v[k], e)));
    *reinterpret_cast<int4 *>(xs + 4 * lane) = make_int4(q[0], q[1], q[2], q[3]);
    if (lane == 0) {
        reinterpret_cast<int32_t *>(ex)[0] = e;
        ex[1] = any_bad ? __builtin_nanf("") : 1.0f;
    }
}

// T[slot][b] for b in [32 BQ, 32 BQ + 32): with v = floor(243 b / 256) the
// code of byte b and d_n its base-3 digits, T = A[d0][d1] + B[d2][d3][d4]
// where A = (d0-1) x0 + (d1-1) x1 and B = ((d2-1) x2 + (d3-1) x3) + (d4-1) x4
// are formed once per thread (9 + 27 sums); the digits are compile-time
// constants of the unrolled loop, so each entry costs one add.
template <int BQ, class T>
__device__ __forceinline__ void lut_build_range(float *tab, int slot, const T (&xv)[5])  // bytes kLutBuildPer * BQ ..
{
    T A[9], B[27];
#pragma unroll
    for (int d0 = 0; d0 < 3; ++d0)
#pragma unroll
        for (int d1 = 0; d1 < 3; ++d1)
            A[3 * d0 + d1] = static_cast<T>(d0 - 1) * xv[0] + static_cast<T>(d1 - 1) * xv[1];
#pragma unroll
    for (int d2 = 0; d2 < 3; ++d2)
#pragma unroll
        for (int d3 = 0; d3 < 3; ++d3) {
            const T c = static_cast<T>(d2 - 1) * xv[2] + static_cast<T>(d3 - 1) * xv[3];
#pragma unroll
            for (int d4 = 0; d4 < 3; ++d4) B[9 * d2 + 3 * d3 + d4] = c + static_cast<T>(d4 - 1) * xv[4];
        }
    const uint32_t base = static_cast<uint32_t>(slot) << 2;  // slot < 64
#pragma unroll
    for (int i = 0; i < kLutBuildPer; ++i) {
        const int b = kLutBuildPer * BQ + i;
        const int v = (243 * b) >> 8;
        *reinterpret_cast<T *>(reinterpret_cast<char *>(tab) + (base | (static_cast<uint32_t>(b) << 8))) =
            A[v / 27] + B[v % 27];
    }
}

// bq (wave-uniform) -> lut_build_range<bq>: the digits of each entry stay
// compile-time constants.
template <int BQ, class T>
__device__ __forceinline__ void lut_build_dispatch(int bq, float *tab, int slot, const T (&xv)[5])
{
    if constexpr (BQ < kLutBuildRanges) {
        if (bq == BQ)
            lut_build_range<BQ, T>(tab, slot, xv);
        else
            lut_build_dispatch<BQ + 1, T>(bq, tab, slot, xv);
    }
}

// One unit = (slice s, matrix mat, 32-row group grp) = tile (grp, s) of
// matrix mat; `un` indexes the units of one slice (matrix-major).  Row
// counts are below 2^20 (checked by the caller), so indices fit in int.
struct LutUnit {
    int mat, grp;
};

__device__ __forceinline__ LutUnit lut_unit(const LutArgs &a, int64_t un)
{
    LutUnit u;
    const int rem = static_cast<int>(un);
    const int groups = static_cast<int>(a.groups);
    u.mat = rem >= groups ? 1 : 0;
    u.grp = rem - u.mat * groups;
    return u;
}

typedef uint32_t lut_u32x4 __attribute__((ext_vector_type(4), aligned(4)));

// U: units per wave.
// One segment of a workgroup's work: units [u0, u1) of slice s, unit
// u0 + w + 8 i going to wave w (i < U).
template <int U, bool W8>
__device__ __forceinline__ void lut_segment(const LutArgs &a, float *tab, float *xs, int s, int64_t u0, int64_t u1)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int64_t k0 = static_cast<int64_t>(s) * kLutSliceW;
    const int kw = static_cast<int>(a.k - k0 < kLutSliceW ? a.k - k0 : kLutSliceW);
    const int nblk = kw / kBlockWeights;
    const int row_l = lane >> 1;  // row of the unit (tile) this lane reads
    const int blk_l = lane & 1;   // block of the slice this lane reads
    const int rho = lut_rho(lane), sig = lut_sig(lane);

    // ---- 1. the table's input is requested before the weights: vector
    // memory returns in order, so anything requested after the weights
    // would wait for all of them.
    SliceX xv;
    if (wave == 0) slice_x_load(a.x, a.signs, a.gain, k0, kw, lane, xv);
    float amax = 0.0f;  // W8: this thread's part of max|x|, 16 bytes per load, all requested at once
    if constexpr (W8) {
        constexpr int kPer = 9;  // float4 loads per thread requested before the reduction (k <= 18432 in one pass)
        lut_f32x4 v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t e = 4 * (tid + static_cast<int64_t>(kLutThreads) * j);
            v[j] = *reinterpret_cast<const lut_f32x4 *>(a.x + (e < a.k ? e : a.k - 4));  // clamped copies repeat
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
        for (int64_t e = 4 * (tid + static_cast<int64_t>(kLutThreads) * kPer); e < a.k; e += 4 * kLutThreads) {
            const lut_f32x4 w = *reinterpret_cast<const lut_f32x4 *>(a.x + e);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3]))));
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. weights of this wave's first kLutEarly units; units up to
    // kLutDepth follow once x has arrived (after the first barrier) and the
    // rest one unit ahead of use during the lookups, so a wave never has more
    // than kLutDepth units in flight.  Requests are served roughly in arrival
    // order: with every unit requested at entry, x's loads queued behind the
    // weights and the table was built later (measured slower); one unit per
    // wave still keeps HBM busy meanwhile.  A lane reads its 28-byte block
    // with two wide loads (16 + 12 bytes; blocks are only dword-aligned,
    // which gfx950 global loads accept) into registers 0..6; register 7 is a
    // zero dword (position 7 of the block, whose columns are zeros).
    uint32_t dat[U][kLutDwords];
    uint32_t scb[U];
    // Unit indices, tile bases and row bases are wave-uniform (scalar
    // registers); a lane adds a 32-bit offset of its own (one address add per
    // unit, no 64-bit index arithmetic in vector registers).
    auto unit_of = [&](int i) { return static_cast<int>(u0) + wave + kLutWaves * i; };
    const uint32_t lane_off = static_cast<uint32_t>(lane * kBlockBytes);
    auto issue = [&](int i) {
        const int un = unit_of(i) < u1 ? unit_of(i) : static_cast<int>(u1) - 1;  // clamped: no branch
        const LutUnit u = lut_unit(a, un);
        // tiled matrices are below 2 GiB (checked by the caller)
        const uint8_t *tile = (u.mat ? a.w1 : a.w0) +
                              (static_cast<uint32_t>(s) * static_cast<uint32_t>(a.groups) +
                               static_cast<uint32_t>(u.grp)) * static_cast<uint32_t>(kTileBytes);
        const lut_u32x4 lo = *reinterpret_cast<const lut_u32x4 *>(tile + lane_off);
        const lut_u32x3 hi = *reinterpret_cast<const lut_u32x3 *>(tile + (lane_off + 16u));
        dat[i][0] = lo.x; dat[i][1] = lo.y; dat[i][2] = lo.z; dat[i][3] = lo.w;
        dat[i][4] = hi.x; dat[i][5] = hi.y; dat[i][6] = hi.z; dat[i][7] = 0u;
    };
    // the scale (the block's upper half dword 6) is kept, then register r
    // receives dword (r + rho) mod 8: rotations by 1 and 2 merged with a
    // lane mask (a select of array elements would become a dynamically
    // indexed, private-memory array)
    auto rotate = [&](int i) {
        scb[i] = dat[i][6] >> 16;
#pragma unroll
        for (int sh = 1; sh <= 2; sh <<= 1) {
            const uint32_t m = (rho & sh) ? 0xffffffffu : 0u;
            uint32_t t[kLutDwords];
#pragma unroll
            for (int j = 0; j < kLutDwords; ++j) t[j] = (dat[i][(j + sh) & 7] & m) | (dat[i][j] & ~m);
#pragma unroll
            for (int j = 0; j < kLutDwords; ++j) dat[i][j] = t[j];
        }
    };
    // wave 0's x requests go out before any wave's weights: a bare barrier
    // (no memory wait), so x is not queued behind the first weight burst
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < (U < kLutEarly ? U : kLutEarly); ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);

    // ---- per-lane lookup constants, formed while x is in flight (they
    // depend on neither x nor the table; formed after the table barrier they
    // held every wave of a SIMD for ~150 VALU operations while the LDS
    // idled).  The address of the lookup of byte c of register r is
    // byte << 8 | column << 2; the four column bytes of a register are packed
    // in P[r] (byte c) and v_perm_b32 inserts the data byte (selector:
    // byte 0 <- P byte c, byte 1 <- data byte (c + sig) & 3, 0, 0).  The
    // packed form is the register's base column replicated into four bytes
    // plus the per-lane byte offsets (no carries: column << 2 < 256).
    uint32_t P[kLutDwords];
    uint32_t S[4];
    uint32_t boff = 0;  // byte c: ((c + sig) & 3) << 2
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t e = static_cast<uint32_t>((c + sig) & 3);
        S[c] = 0x0C0C0000u | (e << 8) | static_cast<uint32_t>(4 + c);
        boff |= (e << 2) << (8 * c);
    }
#pragma unroll
    for (int r = 0; r < kLutDwords; ++r) {
        const int q = (r + rho + 4 * blk_l) & (kLutDwords - 1);  // bank group of dword (r + rho) mod 8
        const uint32_t base = static_cast<uint32_t>(kLutColsPerBlock * blk_l + 4 * q) << 2;
        P[r] = __builtin_amdgcn_perm(base, base, 0x00000000u) + boff;  // base in all four bytes
    }
    // opaque from here on: otherwise the compiler recomputes them next to
    // their uses, after the table barrier
#pragma unroll
    for (int r = 0; r < kLutDwords; ++r) asm volatile("" : "+v"(P[r]));
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(S[c]));
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. x for this slice as int32 q in xs: rotated when signs are
    // given (k % 1024 == 0) and held in fixed point with the slice's power of
    // two 2^-ex; W8: the workgroup's max|x| first, then q = rint(x c)
    // (integers in [-127, 127]) and the step max|x| / 127
    float *red = xs + kLutSliceW;  // kLutWaves floats after the slice
    float step = 1.0f;
    int ex = 0;
    if constexpr (W8) {
        amax = wave_max(amax);
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        float g = 0.0f;
#pragma unroll
        for (int w = 0; w < kLutWaves; ++w) g = fmaxf(g, red[w]);
        // the multiplier rounded once from its exact quotient (the double
        // division is correctly rounded, the conversion rounds to nearest)
        const float c = g > 0.0f ? static_cast<float>(127.0 / static_cast<double>(g)) : 0.0f;
        step = static_cast<float>(static_cast<double>(g) / 127.0);
        if (wave == 0) {
            int32_t qv[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qv[kk] = 4 * lane + kk < kw ? static_cast<int32_t>(rintf(xv.x[0][kk] * c)) : 0;
            *reinterpret_cast<int4 *>(xs + 4 * lane) = make_int4(qv[0], qv[1], qv[2], qv[3]);
        }
    } else {
        if (wave == 0)
            slice_x_store_fixed(slice_x_values(xv, a.signs != nullptr, a.gain != nullptr, k0, kw, lane), lane, xs,
                                red);
    }
    __syncthreads();
    if constexpr (!W8) {
        ex = reinterpret_cast<const int32_t *>(red)[0];
        step = red[1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = kLutEarly; i < (U < kLutDepth ? U : kLutDepth); ++i) issue(i);  // in flight during the build
    __builtin_amdgcn_sched_barrier(0);
    // ---- 4. table: thread = (column, 32-value range of the byte)
    {
        const int bq = tid >> 6;  // 0 .. kLutBuildRanges - 1
        const int col = tid & 63;
        const int blk = col / kLutColsPerBlock;
        const int i = (col - 16 * blk) & (kLutColsPerBlock - 1);  // byte position of this column
        const int32_t *xq = reinterpret_cast<const int32_t *>(xs);
        int32_t xv5[5];
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            const int j = kTritsPerByte * i + n;  // weight index in the block
            xv5[n] = (blk < nblk && i < kTritBytes && j < kBlockWeights) ? xq[blk * kBlockWeights + j] : 0;
        }
        lut_build_dispatch<0, int32_t>(bq, tab, col, xv5);
    }
    rotate(0);
    __syncthreads();
    // the prologue (x, rotation, table) ran at raised wave priority, so a
    // workgroup that starts late on a CU builds its table ahead of the
    // other workgroup's lookups; the lookups run at the normal priority
    __builtin_amdgcn_s_setprio(0);

    // ---- 5. lookups (exact int32 sums, two lookups per v_add3_u32), scale,
    // 2-lane reduction, partial store
    typedef __attribute__((address_space(3))) const int32_t lds_i32;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if (i + kLutDepth < U) issue(i + kLutDepth);  // compile-time condition
        if (i > 0) rotate(i);
        const bool unit_ok = unit_of(i) < u1;  // wave-uniform
        const int un = unit_ok ? unit_of(i) : static_cast<int>(u1) - 1;
        const LutUnit u = lut_unit(a, un);
        const int n = static_cast<int>(a.n);  // rows < 2^20 (checked by the caller)
        const int r0 = u.grp * kLutRows;      // wave-uniform
        const int r = r0 + row_l;
        const bool live = unit_ok && r < n && blk_l < nblk;  // padding rows / blocks contribute nothing
        const float scale = live ? half_bits_to_float(scb[i]) : 0.0f;
        int32_t acc = 0;
#pragma unroll
        for (int j = 0; j < kLutDwords; ++j) {
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
                const uint32_t a0 = __builtin_amdgcn_perm(P[j], dat[i][j], S[c]);
                const uint32_t a1 = __builtin_amdgcn_perm(P[j], dat[i][j], S[c + 1]);
                acc = acc + *reinterpret_cast<lds_i32 *>(static_cast<uintptr_t>(a0)) +
                      *reinterpret_cast<lds_i32 *>(static_cast<uintptr_t>(a1));
            }
        }
        // W8: |acc| <= 26 * 635 < 2^24, exact in fp32; otherwise |acc| < 2^31
        // and the conversion rounds once
        float p = static_cast<float>(acc) * scale;
        const int ip = __builtin_bit_cast(int, p);
        p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ip, ip, 0xB1, 0xF, 0xF, false));  // + lane ^ 1
        if constexpr (!W8) p = ldexpf(p, -ex);
        p *= step;
        float *prow = a.part + ((static_cast<int64_t>(s) * a.nmat + u.mat) * a.n + r0);  // wave-uniform
        if (unit_ok && blk_l == 0 && r < n) prow[row_l] = p;
    }
}

// Grid (workgroups per slice, slices): workgroup (c, s) owns slice s and
// its units [c per_wg, min((c + 1) per_wg, units per slice)), so every
// workgroup has one slice and one table and none holds more than per_wg
// units.  The grid shape carries the partition: no division at entry (the
// 64-bit divisions of an even split cost a dependent chain of scalar and
// reciprocal steps before the first load could be issued).
template <int U, bool W8>
__global__ void __launch_bounds__(kLutThreads, 4) k_matvec_lut(LutArgs a)  // 4 waves per SIMD (1024 threads per CU)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float *tab = reinterpret_cast<float *>(lds);                 // 64 KB table
    float *xs = reinterpret_cast<float *>(lds + kLutTableBytes);  // 256 floats
    const int per_slice = a.nmat * static_cast<int>(a.groups);  // rows < 2^20 (checked by the caller)
    const int u0 = static_cast<int>(blockIdx.x) * a.per_wg;
    const int u1 = u0 + a.per_wg < per_slice ? u0 + a.per_wg : per_slice;
    __builtin_amdgcn_s_setprio(3);
    if (u0 < u1) lut_segment<U, W8>(a, tab, xs, static_cast<int>(blockIdx.y), u0, u1);  // workgroup-uniform
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

int64_t lut_nslices(int64_t k) { return (k + kLutSliceW - 1) / kLutSliceW; }

size_t lut_part_floats(int64_t n, int nmat, int64_t k) { return static_cast<size_t>(lut_nslices(k) * nmat * n); }

// Up to two workgroups per CU (at most one per 8 units), the same number cs
// of workgroups for every slice, each taking per_wg = ceil(units / cs)
// consecutive units; U = units per wave of a full workgroup, chunks = the
// workgroups per slice that get units.
struct LutPlan {
    int U;
    int per_wg;
    int64_t chunks;
};

static LutPlan lut_plan(int64_t per_slice, int64_t nslices)
{
    const int64_t total = per_slice * nslices;
    int64_t wgs = kLutWgPerCu * static_cast<int64_t>(device_cus());
    if (wgs > total / kLutWaves) wgs = total / kLutWaves;
    int64_t cs = wgs / nslices;
    if (cs < 1) cs = 1;
    // at most 6 units per wave: a wave holds all of its units' weights in
    // registers, and 8 would not fit beside the rotation's inputs
    static const int kUs[] = {1, 2, 3, 4, 6};
    int U = 0;
    int64_t per_wg = 0;
    for (;;) {
        per_wg = (per_slice + cs - 1) / cs;
        const int64_t need = (per_wg + kLutWaves - 1) / kLutWaves;
        for (int cand : kUs)
            if (cand >= need) {
                U = cand;
                break;
            }
        if (U != 0) break;
        ++cs;  // parts above 48 units: more workgroups per slice
    }
    return LutPlan{U, static_cast<int>(per_wg), (per_slice + per_wg - 1) / per_wg};
}

template <int U, bool W8>
static hipError_t lut_launch(const LutArgs &a, int64_t chunks, hipStream_t st)
{
    static std::atomic<uint64_t> lds_done{0};
    const size_t lds = kLutTableBytes + (kLutSliceW + kLutWaves) * sizeof(float);
    const hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void *>(&k_matvec_lut<U, W8>), static_cast<int>(lds), lds_done);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.nslices));
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL((k_matvec_lut<U, W8>), grid, dim3(kLutThreads), static_cast<uint32_t>(lds), st, pe.start,
                              pe.stop, 0u, a);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL((k_matvec_lut<U, W8>), grid, dim3(kLutThreads), lds, st, a);
    }
    return hipGetLastError();
}

template <bool W8>
static hipError_t lut_dispatch(const LutArgs &a, int U, int64_t chunks, hipStream_t s)
{
    switch (U) {
        case 1: return lut_launch<1, W8>(a, chunks, s);
        case 2: return lut_launch<2, W8>(a, chunks, s);
        case 3: return lut_launch<3, W8>(a, chunks, s);
        case 4: return lut_launch<4, W8>(a, chunks, s);
        default: return lut_launch<6, W8>(a, chunks, s);
    }
}

hipError_t launch_matvec_lut(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k,
                             const float *x, const float *signs, const float *gain, float *part, hipStream_t s,
                             bool w8)
{
    if (n == 0) return hipSuccess;
    LutArgs a{};
    a.w0 = w0;
    a.w1 = w1;
    a.n = n;
    a.k = k;
    a.nmat = nmat;
    a.nslices = static_cast<int>(lut_nslices(k));
    a.groups = (n + kLutRows - 1) / kLutRows;
    a.x = x;
    a.signs = w8 ? nullptr : signs;
    a.gain = w8 ? nullptr : gain;
    a.part = part;
    const LutPlan pl = lut_plan(static_cast<int64_t>(nmat) * a.groups, a.nslices);
    a.per_wg = pl.per_wg;
    return w8 ? lut_dispatch<true>(a, pl.U, pl.chunks, s) : lut_dispatch<false>(a, pl.U, pl.chunks, s);
}

// ---------------------------------------------------------------------------
// The pages' own decode ("A 27B model in 5.5 GB: Bonsai ternary on Ferrox,
// locally", "What Ferrox does with it": eight lanes share one 128-weight
// block, each lane owns whole bytes, every block is read once, and each trit
// is peeled on the float pipeline as floor(3^(n+1) u) - 3 floor(3^n u),
// u = byte / 256), on the same tiled layout, K-slices, rotation prologue and
// split-K partials as the lookup kernel above, so the two decodes differ only
// in how a block's dot product is formed.
//
// Lane l: b = l / 32 is the block of the slice, r = (l / 8) mod 4 a row of
// the step's four, j = l mod 8 the dword of the block the lane owns (bytes
// 4j .. 4j + 3, i.e. weights 20j .. 20j + 19; dword 6 holds the last two
// trit bytes and the scale; lane 7 owns nothing).  A step covers rows
// 4 st .. 4 st + 3 of a tile, i.e. its blocks 8 st .. 8 st + 7: one dword
// load per lane reads 224 contiguous bytes.  A lane keeps the 20 rotated
// activations of its bytes in registers for the whole kernel (zeros for
// weights past the block and for lane 7), so every step is
//   sum_n (digit_n - 1) x_n = sum_n digit_n x_n - sum_n x_n
// over its bytes, then a sum over the eight lanes (DPP), times the scale
// (lane 6), plus the other block of the row (lane l ^ 32).  Cost on gfx950:
// about 20 VALU operations per byte (byte to float, five products and
// floors, four digit differences, five FMAs), i.e. 4 per weight, against
// the lookup kernel's 2 per five weights.
// ---------------------------------------------------------------------------
constexpr int kPeelSteps = kLutRows / 4;  // 8 steps of 4 rows x 2 blocks per tile

template <int U>
__device__ __forceinline__ void peel_segment(const LutArgs &a, float *xs, int s, int64_t u0, int64_t u1)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t k0 = static_cast<int64_t>(s) * kLutSliceW;
    const int kw = static_cast<int>(a.k - k0 < kLutSliceW ? a.k - k0 : kLutSliceW);
    const int nblk = kw / kBlockWeights;
    const int hb = lane >> 5;        // block of the slice
    const int rr = (lane >> 3) & 3;  // row of the step
    const int jd = lane & 7;         // owned dword (7: none)
    const int jl = jd < kBlockDwords ? jd : kBlockDwords - 1;  // dword actually loaded (lane 7 repeats 6)

    // ---- 1. x for the slice (wave 0), requested before any weights
    SliceX xv;
    if (wave == 0) slice_x_load(a.x, a.signs, a.gain, k0, kw, lane, xv);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. weights: one dword per lane and step, two units in flight
    uint32_t dat[2][kPeelSteps];
    auto unit_of = [&](int i) { return u0 + wave + static_cast<int64_t>(kLutWaves) * i; };
    auto issue = [&](int i) {
        const int64_t un = unit_of(i) < u1 ? unit_of(i) : u1 - 1;  // clamped: no branch
        const LutUnit u = lut_unit(a, un);
        const uint8_t *tile = (u.mat ? a.w1 : a.w0) +
                              (static_cast<uint32_t>(s) * static_cast<uint32_t>(a.groups) +
                               static_cast<uint32_t>(u.grp)) * static_cast<uint32_t>(kTileBytes);
#pragma unroll
        for (int st = 0; st < kPeelSteps; ++st)
            dat[i & 1][st] = *reinterpret_cast<const uint32_t *>(
                tile + (2 * (4 * st + rr) + hb) * kBlockBytes + 4 * jl);
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. the slice's x (times the gain), rotated
    if (wave == 0) slice_x_store(xv, a.signs != nullptr, a.gain != nullptr, k0, kw, lane, xs);
    __syncthreads();

    // ---- 4. this lane's 20 activations (zero past the block, for lane 7
    // and for a block the slice does not have) and their sum
    float xr[20];
    float xsum = 0.0f;
#pragma unroll
    for (int n = 0; n < 20; ++n) {
        const int w = 20 * jd + n;  // weight index in the block
        xr[n] = (hb < nblk && jd < kBlockDwords && w < kBlockWeights) ? xs[kBlockWeights * hb + (w < kBlockWeights ? w : 0)]
                                                                     : 0.0f;
        xsum += xr[n];
    }

    // ---- 5. per unit: 8 steps of peel, 8-lane sum, scale, the row's two blocks
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if (i + 1 < U) issue(i + 1);  // compile-time condition
        const bool unit_ok = unit_of(i) < u1;  // wave-uniform
        const int64_t un = unit_ok ? unit_of(i) : u1 - 1;
        const LutUnit u = lut_unit(a, un);
#pragma unroll
        for (int st = 0; st < kPeelSteps; ++st) {
            const uint32_t d = dat[i & 1][st];
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const Peel5 pd = peel5(static_cast<float>((d >> (8 * c)) & 0xffu));
                acc = fmaf(pd.d0, xr[5 * c + 0], acc);
                acc = fmaf(pd.d1, xr[5 * c + 1], acc);
                acc = fmaf(pd.d2, xr[5 * c + 2], acc);
                acc = fmaf(pd.d3, xr[5 * c + 3], acc);
                acc = fmaf(pd.d4, xr[5 * c + 4], acc);
            }
            float t = acc - xsum;
            // sum over the 8 lanes of the block: mirror within 8, then quad swaps
            int it = __builtin_bit_cast(int, t);
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(it, it, 0x141, 0xF, 0xF, false));
            it = __builtin_bit_cast(int, t);
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(it, it, 0xB1, 0xF, 0xF, false));
            it = __builtin_bit_cast(int, t);
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(it, it, 0x4E, 0xF, 0xF, false));
            const int r = u.grp * kLutRows + 4 * st + rr;
            const bool live = unit_ok && r < a.n && hb < nblk;
            float v = live ? t * half_bits_to_float(d >> 16) : 0.0f;  // lane 6 holds the scale
            // + the row's other block (lane ^ 32)
            const uint32_t uv = __builtin_bit_cast(uint32_t, v);
            const auto sw = __builtin_amdgcn_permlane32_swap(uv, uv, false, false);
            const uint32_t s0 = sw[0], s1 = sw[1];
            v = __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
            if (jd == kBlockDwords - 1 && hb == 0 && unit_ok && r < a.n)
                a.part[(static_cast<int64_t>(s) * a.nmat + u.mat) * a.n + r] = v;
        }
    }
}

template <int U>
__global__ void __launch_bounds__(kLutThreads) k_matvec_peel(LutArgs a)
{
    __shared__ __attribute__((aligned(16))) float xs[kLutSliceW];
    const int per_slice = a.nmat * static_cast<int>(a.groups);
    const int u0 = static_cast<int>(blockIdx.x) * a.per_wg;
    const int u1 = u0 + a.per_wg < per_slice ? u0 + a.per_wg : per_slice;
    if (u0 < u1) peel_segment<U>(a, xs, static_cast<int>(blockIdx.y), u0, u1);
}

template <int U>
static hipError_t peel_launch(const LutArgs &a, int64_t chunks, hipStream_t st)
{
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.nslices));
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL(k_matvec_peel<U>, grid, dim3(kLutThreads), 0u, st, pe.start, pe.stop, 0u, a);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL(k_matvec_peel<U>, grid, dim3(kLutThreads), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_matvec_peel(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k, const float *x,
                              const float *signs, const float *gain, float *part, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    LutArgs a{};
    a.w0 = w0;
    a.w1 = w1;
    a.n = n;
    a.k = k;
    a.nmat = nmat;
    a.nslices = static_cast<int>(lut_nslices(k));
    a.groups = (n + kLutRows - 1) / kLutRows;
    a.x = x;
    a.signs = signs;
    a.gain = gain;
    a.part = part;
    const LutPlan pl = lut_plan(static_cast<int64_t>(nmat) * a.groups, a.nslices);
    a.per_wg = pl.per_wg;
    switch (pl.U) {
        case 1: return peel_launch<1>(a, pl.chunks, s);
        case 2: return peel_launch<2>(a, pl.chunks, s);
        case 3: return peel_launch<3>(a, pl.chunks, s);
        case 4: return peel_launch<4>(a, pl.chunks, s);
        default: return peel_launch<6>(a, pl.chunks, s);
    }
}

// ---------------------------------------------------------------------------
// PQ2_0 decode matvec ("Why I Am Building Another Inference Engine", Level 2:
// two bits per ternary weight and a 16-bit scale for every 128 weights).  The
// same table scheme: a byte holds four 2-bit codes, so a 2-block slice has
// 64 byte slots and T[slot][b] = sum_f w(field f of b) xr[k(slot, f)], with
// w(q) = q - 1 and w(3) = 0.  What differs from PTQ1_0:
//   - a lane's block is 32 code bytes, read with two 16-byte loads from its
//     tile record, and its scale comes from the tile's scale area;
//   - the 64 slots fill the table's 64 columns (block b's slot p at column
//     32 b + (p + 16 b) mod 32), and lane 2i + b rotates its 8 dwords by
//     rho = (i / 4) mod 4 and its bytes by sig = i mod 4, as in the PTQ1_0
//     kernel: at lookup (j, c) the 16 block-0 lanes of a half-wave read the
//     banks of dwords j .. j + 3 (mod 8) and the block-1 lanes, 16 banks
//     further, the other 16, so no two lanes of a half-wave share a bank;
//   - 32 lookups per block and no scale-byte lookups.
// The table is int32 over the slice's fixed-point q (slice_x_store_fixed),
// as in the PTQ1_0 kernel (|T| <= 4 * 2^23, a block's 32 entries < 2^31).
// Partials and their sums are those of the PTQ1_0 kernel.
// ---------------------------------------------------------------------------
constexpr int kPq2Slots = kLutBlocks * kPq2CodeBytes;  // 64
constexpr int kPq2Dwords = kPq2CodeBytes / 4;          // 8
static_assert(kPq2Slots * 256 * 4 == kLutTableBytes, "the PQ2_0 table fills the 64 KB array");

struct Pq2Args {
    const uint8_t *w0, *w1;  // PQ2_0 tiled [n][k]; w1 used when nmat == 2
    int64_t n, k;
    int nmat, nslices;
    int64_t groups;          // ceil(n / 32)
    int per_wg;
    const float *x, *signs;  // x [k], rotated here when signs != nullptr
    const float *gain;       // [k] or nullptr: x is used as gain * x
    float *part;             // [nslices][nmat][n]
};

__device__ __forceinline__ int pq2_rho(int lane) { return (lane >> 3) & 3; }
__device__ __forceinline__ int pq2_sig(int lane) { return (lane >> 1) & 3; }

// d[j] <- d[(j + rho) mod 8]: conditional rotations by 1 and 2
__device__ __forceinline__ void pq2_rotate(uint32_t (&d)[kPq2Dwords], int rho)
{
#pragma unroll
    for (int sh = 1; sh <= 2; sh <<= 1) {
        const uint32_t m = (rho & sh) ? 0xffffffffu : 0u;
        uint32_t t[kPq2Dwords];
#pragma unroll
        for (int j = 0; j < kPq2Dwords; ++j) t[j] = (d[(j + sh) % kPq2Dwords] & m) | (d[j] & ~m);
#pragma unroll
        for (int j = 0; j < kPq2Dwords; ++j) d[j] = t[j];
    }
}

// T[slot][b] for b in [32 BQ, 32 BQ + 32): b = f0 | f1 << 2 | f2 << 4 | f3 << 6;
// T = A[b & 15] + B[b >> 4] with A = w(f0) x0 + w(f1) x1, B = w(f2) x2 + w(f3) x3.
template <int BQ>
__device__ __forceinline__ void pq2_build_range(float *tab, int col, const int32_t (&xv)[4])
{
    int32_t A[16], B[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int q0 = q & 3, q1 = q >> 2;
        const int32_t w0 = q0 == 3 ? 0 : q0 - 1, w1 = q1 == 3 ? 0 : q1 - 1;
        A[q] = w0 * xv[0] + w1 * xv[1];
        B[q] = w0 * xv[2] + w1 * xv[3];
    }
    const uint32_t base = static_cast<uint32_t>(col) << 2;  // col < 64
#pragma unroll
    for (int i = 0; i < kLutBuildPer; ++i) {
        const int b = kLutBuildPer * BQ + i;
        *reinterpret_cast<int32_t *>(reinterpret_cast<char *>(tab) + (base | (static_cast<uint32_t>(b) << 8))) =
            A[b & 15] + B[b >> 4];
    }
}

template <int BQ>
__device__ __forceinline__ void pq2_build_dispatch(int bq, float *tab, int slot, const int32_t (&xv)[4])
{
    if constexpr (BQ < kLutBuildRanges) {
        if (bq == BQ)
            pq2_build_range<BQ>(tab, slot, xv);
        else
            pq2_build_dispatch<BQ + 1>(bq, tab, slot, xv);
    }
}

template <int U>
__device__ __forceinline__ void pq2_segment(const Pq2Args &a, float *tab, float *xs, int s, int u0, int u1)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t k0 = static_cast<int64_t>(s) * kLutSliceW;
    const int kw = static_cast<int>(a.k - k0 < kLutSliceW ? a.k - k0 : kLutSliceW);
    const int nblk = kw / kBlockWeights;
    const int row_l = lane >> 1;
    const int blk_l = lane & 1;
    const int rho = pq2_rho(lane), sig = pq2_sig(lane);

    // ---- 1. x for the slice's rotation, requested before any weights
    SliceX xv;
    if (wave == 0) slice_x_load(a.x, a.signs, a.gain, k0, kw, lane, xv);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. weights: kLutEarly units before x arrives, up to kLutDepth after
    uint32_t dat[U][kPq2Dwords];
    uint32_t scw[U];
    auto unit_of = [&](int i) { return u0 + wave + kLutWaves * i; };
    auto issue = [&](int i) {
        const int un = unit_of(i) < u1 ? unit_of(i) : u1 - 1;  // clamped: no branch
        const int mat = un >= static_cast<int>(a.groups) ? 1 : 0;
        const int grp = un - mat * static_cast<int>(a.groups);
        // tiled matrices are below 2 GiB (checked by the caller)
        const uint8_t *tb = (mat ? a.w1 : a.w0) + (static_cast<uint32_t>(s) * static_cast<uint32_t>(a.groups) +
                                                   static_cast<uint32_t>(grp)) * static_cast<uint32_t>(kPq2TileBytes);
        const lut_u32x4 lo = *reinterpret_cast<const lut_u32x4 *>(tb + lane * kPq2CodeBytes);
        const lut_u32x4 hi = *reinterpret_cast<const lut_u32x4 *>(tb + lane * kPq2CodeBytes + 16);
        dat[i][0] = lo.x; dat[i][1] = lo.y; dat[i][2] = lo.z; dat[i][3] = lo.w;
        dat[i][4] = hi.x; dat[i][5] = hi.y; dat[i][6] = hi.z; dat[i][7] = hi.w;
        scw[i] = *reinterpret_cast<const uint32_t *>(tb + kPq2TileCodeBytes + 4 * (lane >> 1));  // scales of 2i, 2i+1
    };
    __builtin_amdgcn_s_barrier();  // wave 0's x requests go first (as in the PTQ1_0 kernel)
#pragma unroll
    for (int i = 0; i < (U < kLutEarly ? U : kLutEarly); ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);

    // ---- per-lane lookup constants (as in the PTQ1_0 kernel; slot < 64)
    uint32_t P[kPq2Dwords];
    uint32_t S[4];
    uint32_t boff = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t e = static_cast<uint32_t>((c + sig) & 3);
        S[c] = 0x0C0C0000u | (e << 8) | static_cast<uint32_t>(4 + c);
        boff |= (e << 2) << (8 * c);
    }
#pragma unroll
    for (int j = 0; j < kPq2Dwords; ++j) {
        const int q = (j + rho + 4 * blk_l) & (kPq2Dwords - 1);  // bank group of dword (j + rho) mod 8
        const uint32_t base = static_cast<uint32_t>(kPq2CodeBytes * blk_l + 4 * q) << 2;
        P[j] = __builtin_amdgcn_perm(base, base, 0x00000000u) + boff;
    }
#pragma unroll
    for (int j = 0; j < kPq2Dwords; ++j) asm volatile("" : "+v"(P[j]));
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(S[c]));
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. the slice's x (times the gain), rotated, in fixed point
    float *ex = xs + kLutSliceW;
    if (wave == 0)
        slice_x_store_fixed(slice_x_values(xv, a.signs != nullptr, a.gain != nullptr, k0, kw, lane), lane, xs, ex);
    __syncthreads();
    const int e2 = reinterpret_cast<const int32_t *>(ex)[0];
    const float sfix = ex[1];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = kLutEarly; i < (U < kLutDepth ? U : kLutDepth); ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);
    // ---- 4. table: thread = (slot, 32-value range of the byte)
    {
        const int bq = tid >> 6;
        const int col = tid & 63;  // all 64 columns are used
        const int blk = col / kPq2CodeBytes;
        const int i = (col - 16 * blk) & (kPq2CodeBytes - 1);  // code-byte slot of this column
        const int32_t *xq = reinterpret_cast<const int32_t *>(xs);
        int32_t xv[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) xv[f] = blk < nblk ? xq[blk * kBlockWeights + kPq2CodesPerByte * i + f] : 0;
        pq2_build_dispatch<0>(bq, tab, col, xv);
    }
    pq2_rotate(dat[0], rho);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);  // the prologue ran at raised priority, as in the PTQ1_0 kernel

    // ---- 5. lookups (int32, two per v_add3_u32), scale, 2-lane reduction,
    // partial store
    typedef __attribute__((address_space(3))) const int32_t lds_i32;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if (i + kLutDepth < U) issue(i + kLutDepth);
        const bool unit_ok = unit_of(i) < u1;
        const int un = unit_ok ? unit_of(i) : u1 - 1;
        const int mat = un >= static_cast<int>(a.groups) ? 1 : 0;
        const int r = (un - mat * static_cast<int>(a.groups)) * kLutRows + row_l;
        const bool live = unit_ok && r < a.n && blk_l < nblk;
        const uint32_t sh = blk_l ? (scw[i] >> 16) : (scw[i] & 0xffffu);
        const float scale = live ? half_bits_to_float(sh) : 0.0f;
        if (i > 0) pq2_rotate(dat[i], rho);
        int32_t acc = 0;
#pragma unroll
        for (int j = 0; j < kPq2Dwords; ++j) {
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
                const uint32_t a0 = __builtin_amdgcn_perm(P[j], dat[i][j], S[c]);
                const uint32_t a1 = __builtin_amdgcn_perm(P[j], dat[i][j], S[c + 1]);
                acc = acc + *reinterpret_cast<lds_i32 *>(static_cast<uintptr_t>(a0)) +
                      *reinterpret_cast<lds_i32 *>(static_cast<uintptr_t>(a1));
            }
        }
        float p = static_cast<float>(acc) * scale;
        const int ip = __builtin_bit_cast(int, p);
        p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ip, ip, 0xB1, 0xF, 0xF, false));  // + lane ^ 1
        p = ldexpf(p, -e2) * sfix;
        if (unit_ok && blk_l == 0 && r < a.n) a.part[(static_cast<int64_t>(s) * a.nmat + mat) * a.n + r] = p;
    }
}

template <int U>
__global__ void __launch_bounds__(kLutThreads, 4) k_pq2_matvec(Pq2Args a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float *tab = reinterpret_cast<float *>(lds);
    float *xs = reinterpret_cast<float *>(lds + kLutTableBytes);
    const int per_slice = a.nmat * static_cast<int>(a.groups);
    const int u0 = static_cast<int>(blockIdx.x) * a.per_wg;
    const int u1 = u0 + a.per_wg < per_slice ? u0 + a.per_wg : per_slice;
    __builtin_amdgcn_s_setprio(3);  // prologue at raised priority (lowered before the lookups)
    if (u0 < u1) pq2_segment<U>(a, tab, xs, static_cast<int>(blockIdx.y), u0, u1);
}

template <int U>
static hipError_t pq2_launch(const Pq2Args &a, int64_t chunks, hipStream_t st)
{
    static std::atomic<uint64_t> lds_done{0};
    // the table, the slice's q and the fixed-point exponent and factor
    const size_t lds = kLutTableBytes + (kLutSliceW + kLutWaves) * sizeof(float);
    const hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void *>(&k_pq2_matvec<U>), static_cast<int>(lds), lds_done);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.nslices));
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL(k_pq2_matvec<U>, grid, dim3(kLutThreads), static_cast<uint32_t>(lds), st, pe.start,
                              pe.stop, 0u, a);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL(k_pq2_matvec<U>, grid, dim3(kLutThreads), lds, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_pq2_matvec(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k, const float *x,
                             const float *signs, const float *gain, float *part, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    Pq2Args a{};
    a.w0 = w0;
    a.w1 = w1;
    a.nmat = nmat;
    a.gain = gain;
    a.n = n;
    a.k = k;
    a.nslices = static_cast<int>(lut_nslices(k));
    a.groups = (n + kLutRows - 1) / kLutRows;
    a.x = x;
    a.signs = signs;
    a.part = part;
    const LutPlan pl = lut_plan(static_cast<int64_t>(nmat) * a.groups, a.nslices);
    a.per_wg = pl.per_wg;
    switch (pl.U) {
        case 1: return pq2_launch<1>(a, pl.chunks, s);
        case 2: return pq2_launch<2>(a, pl.chunks, s);
        case 3: return pq2_launch<3>(a, pl.chunks, s);
        case 4: return pq2_launch<4>(a, pl.chunks, s);
        default: return pq2_launch<6>(a, pl.chunks, s);
    }
}

// ---------------------------------------------------------------------------
// Split-K sums.  Every partial of a thread is requested before any is
// added (clamped indices: no branch around the loads); rows are summed in
// slice order, so results are deterministic.
// ---------------------------------------------------------------------------
constexpr int kSumPer = 24;       // partials per thread per round
constexpr int kSumThreads = 256;

// y[r] = (residual ? residual[r] : 0) + sum_s part[s][r].  T threads per
// row: lane = j * (64 / T) + i sums slices [j ns / T, (j + 1) ns / T) of row
// i of the wave's 64 / T rows (consecutive lanes read consecutive rows), and
// the T sums are combined in fixed order.
template <int T>
__global__ void __launch_bounds__(kSumThreads) k_lut_sum_rows(const float *__restrict__ part, int64_t n, int ns,
                                                              const float *residual, float *y)
{
    constexpr int kRowsPerWave = kWave / T;
    const int lane = threadIdx.x & (kWave - 1);
    const int j = lane / kRowsPerWave;
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * (kSumThreads / kWave) + threadIdx.x / kWave) * kRowsPerWave +
                      lane % kRowsPerWave;
    const int64_t rc = r < n ? r : n - 1;
    const int q_lo = static_cast<int>(static_cast<int64_t>(j) * ns / T);
    const int q_hi = static_cast<int>(static_cast<int64_t>(j + 1) * ns / T);
    // the residual is requested with the partials (after the sum it would
    // cost a second round trip to memory)
    const float res = residual != nullptr ? residual[rc] : 0.0f;
    float t = 0.0f;
    for (int q0 = q_lo; q0 < q_hi; q0 += kSumPer) {
        float v[kSumPer];
#pragma unroll
        for (int c = 0; c < kSumPer; ++c) {
            const int q = q0 + c < q_hi ? q0 + c : q_hi - 1;
            v[c] = part[static_cast<int64_t>(q) * n + rc];
        }
#pragma unroll
        for (int c = 0; c < kSumPer; ++c)
            if (q0 + c < q_hi) t += v[c];
    }
    // lower slice range first: the same order in every lane
    if constexpr (T == 4) t = lane_pair_sum<16>(t);
    if constexpr (T >= 2) t = lane_pair_sum<32>(t);
    if (j == 0 && r < n) y[r] = residual ? res + t : t;
}

hipError_t launch_lut_sum_rows(const float *part, int64_t n, int64_t k, const float *residual, float *y,
                               hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const int ns = static_cast<int>(lut_nslices(k));
    const int T = ns <= kSumPer ? 1 : (ns <= 2 * kSumPer ? 2 : 4);
    const int64_t rows_per_wg = static_cast<int64_t>(kSumThreads) / T;
    const dim3 grid(static_cast<unsigned>((n + rows_per_wg - 1) / rows_per_wg));
    switch (T) {
        case 1: hipLaunchKernelGGL(k_lut_sum_rows<1>, grid, dim3(kSumThreads), 0, s, part, n, ns, residual, y); break;
        case 2: hipLaunchKernelGGL(k_lut_sum_rows<2>, grid, dim3(kSumThreads), 0, s, part, n, ns, residual, y); break;
        default: hipLaunchKernelGGL(k_lut_sum_rows<4>, grid, dim3(kSumThreads), 0, s, part, n, ns, residual, y); break;
    }
    return hipGetLastError();
}

// Gate/up epilogue, T threads per row as in k_lut_sum_rows (thread j sums
// slices [j ns / T, (j + 1) ns / T) of both matrices):
//   g, u = a * sum_s part[s][0][r], a * sum_s part[s][1][r]  (a = RMS scale
//   of x_rms [d], or 1 when x_rms == nullptr), h = silu(g) * u; any of g, u,
//   h may be nullptr.  Every workgroup computes a itself (d values from L2).
template <int T>
__global__ void __launch_bounds__(kSumThreads) k_lut_gate_up_sum(
    const float *__restrict__ part, int64_t f, int ns, const float *__restrict__ x_rms, int64_t d, float rms_eps,
    float *g, float *u, float *h)
{
    constexpr int kRowsPerWave = kWave / T;
    constexpr int kRmsPer = 24;  // RMS inputs per thread requested up front (d <= 6144), any rest below
    __shared__ float red[kSumThreads / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int j = lane / kRowsPerWave;
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * (kSumThreads / kWave) + wave) * kRowsPerWave +
                      lane % kRowsPerWave;
    const int64_t rc = r < f ? r : f - 1;
    float rv[kRmsPer];
    if (x_rms != nullptr) {
#pragma unroll
        for (int c = 0; c < kRmsPer; ++c) {
            const int64_t i = tid + static_cast<int64_t>(c) * kSumThreads;
            rv[c] = x_rms[i < d ? i : d - 1];
        }
    }
    const int q_lo = static_cast<int>(static_cast<int64_t>(j) * ns / T);
    const int q_hi = static_cast<int>(static_cast<int64_t>(j + 1) * ns / T);
    float tg = 0.0f, tu = 0.0f;
    for (int q0 = q_lo; q0 < q_hi; q0 += kSumPer / 2) {
        float vg[kSumPer / 2], vu[kSumPer / 2];
#pragma unroll
        for (int c = 0; c < kSumPer / 2; ++c) {
            const int q = q0 + c < q_hi ? q0 + c : q_hi - 1;
            vg[c] = part[(2 * static_cast<int64_t>(q)) * f + rc];
            vu[c] = part[(2 * static_cast<int64_t>(q) + 1) * f + rc];
        }
#pragma unroll
        for (int c = 0; c < kSumPer / 2; ++c) {
            if (q0 + c < q_hi) {
                tg += vg[c];
                tu += vu[c];
            }
        }
    }
    // lower slice range first: the same order in every lane
    if constexpr (T == 4) {
        tg = lane_pair_sum<16>(tg);
        tu = lane_pair_sum<16>(tu);
    }
    if constexpr (T >= 2) {
        tg = lane_pair_sum<32>(tg);
        tu = lane_pair_sum<32>(tu);
    }
    float a = 1.0f;
    if (x_rms != nullptr) {
        float sq = 0.0f;
#pragma unroll
        for (int c = 0; c < kRmsPer; ++c)
            if (tid + static_cast<int64_t>(c) * kSumThreads < d) sq = fmaf(rv[c], rv[c], sq);
        for (int64_t i = tid + static_cast<int64_t>(kRmsPer) * kSumThreads; i < d; i += kSumThreads)
            sq = fmaf(x_rms[i], x_rms[i], sq);
        sq = wave_sum(sq);
        if (lane == 0) red[wave] = sq;
        __syncthreads();
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kSumThreads / kWave; ++w) t += red[w];
        a = 1.0f / sqrtf(t / static_cast<float>(d) + rms_eps);
    }
    if (j == 0 && r < f) {
        const float gv = tg * a, uv = tu * a;
        if (g) g[r] = gv;
        if (u) u[r] = uv;
        if (h) h[r] = gv / (1.0f + expf(-gv)) * uv;
    }
}

hipError_t launch_lut_gate_up_sum(const float *part, int64_t f, int64_t d_in, const float *x_rms, int64_t d_rms,
                                  float rms_eps, float *g, float *u, float *h, hipStream_t s)
{
    if (f == 0) return hipSuccess;
    const int ns = static_cast<int>(lut_nslices(d_in));
    const int T = ns <= kSumPer / 2 ? 1 : (ns <= kSumPer ? 2 : 4);
    const int64_t rows_per_wg = static_cast<int64_t>(kSumThreads) / T;
    const dim3 grid(static_cast<unsigned>((f + rows_per_wg - 1) / rows_per_wg));
    switch (T) {
        case 1:
            hipLaunchKernelGGL(k_lut_gate_up_sum<1>, grid, dim3(kSumThreads), 0, s, part, f, ns, x_rms, d_rms, rms_eps,
                               g, u, h);
            break;
        case 2:
            hipLaunchKernelGGL(k_lut_gate_up_sum<2>, grid, dim3(kSumThreads), 0, s, part, f, ns, x_rms, d_rms, rms_eps,
                               g, u, h);
            break;
        default:
            hipLaunchKernelGGL(k_lut_gate_up_sum<4>, grid, dim3(kSumThreads), 0, s, part, f, ns, x_rms, d_rms, rms_eps,
                               g, u, h);
            break;
    }
    return hipGetLastError();
}

}  // namespace ptq1
