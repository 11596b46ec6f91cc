// gemm.hip -- multi-token prefill: PTQ1_0 weights decoded into LDS as exact
// bf16 trits, activations rotated and rounded to bf16, bf16 MFMA with fp32
// accumulation and the per-block scale applied in fp32.
//
// "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally":
//   - "What Ferrox does with it": a GEMM for prefill whose weight tiles are
//     decoded from the packed trits;
//   - "What Bonsai is": activations rotated before every folded matmul.
// Each 128-weight block's MFMA partial sum is multiplied by that block's
// scale in fp32 (never folded into bf16), so the only rounding beyond fp32
// is the bf16 rounding of the rotated activations.
//
// K order inside a block.  A dot product does not depend on the order in
// which K is summed, so both operands are stored in one fixed permutation of
// the block's 128 positions that makes the trit decode cheap: MFMA K
// position kappa = 8 f + j (fragment f = 0..15, element j = 0..7) carries
//   f < 15:  digit d = f % 5 of byte 8 (f / 5) + j   (weight 5 byte + d),
//   f = 15:  weight 120 + j   (bytes 24 and 25 in natural order).
// One fragment is then "digit d of eight consecutive bytes", which a table
// read per byte and one v_perm per pair of bytes produce directly.  MFMA
// step s (0..7) takes fragment s in lanes 0-31 and fragment
// kHiFrag[s] = 10, 11, 12, 13, 14, 8, 9, 15 in lanes 32-63: then a half-wave
// only ever needs 16-20 bytes of a block (lanes 0-31 bytes 0-15, lanes
// 32-63 bytes 8-27) and both halves read the same digit position in steps
// 0-4.  The activation side is written in the same order by the prep kernel.
#include <hip/hip_ext.h>

#include "ptq1_device.h"
#include "ptq1_launch.h"

namespace ptq1 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t gm_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t gm_u32x4 __attribute__((ext_vector_type(4)));
typedef float gm_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t gm_u32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t gm_u32x4a __attribute__((ext_vector_type(4), aligned(4)));

__host__ __device__ constexpr int gemm_hi_frag(int step)
{
    return step < 5 ? 10 + step : (step == 5 ? 8 : (step == 6 ? 9 : 15));
}

// Weight index (0..127 inside the block) held at MFMA K position kappa.
__host__ __device__ constexpr int gemm_kperm(int kappa)
{
    return (kappa >> 3) == 15 ? kappa : 5 * (8 * ((kappa >> 3) / 5) + (kappa & 7)) + (kappa >> 3) % 5;
}

// K order inside a block for the int8 MFMA (v_mfma_i32_32x32x32_i8, four
// steps of K = 32 per block; lane half h of step s supplies K positions
// 32 s + 16 h .. 32 s + 16 h + 15 as four dwords q of four bytes j, and
// t = 4 s + q):
//   t < 12:  digit j of byte 12 h + t              (weight 5 (12 h + t) + j)
//   t = 12:  weight 120 + 4 h + j                   (bytes 24 and 25)
//   t > 12:  digit 4 of byte 12 h + 4 (t - 13) + j
// so each of a lane's dwords with t < 12 is one table entry (digits 0-3 of
// one byte), and those with t > 12 gather digit 4 of four bytes.
__host__ __device__ constexpr int gemm_i8_kperm(int kappa)
{
    const int h = (kappa >> 4) & 1, t = 4 * (kappa >> 5) + ((kappa >> 2) & 3), j = kappa & 3;
    return t < 12 ? 5 * (12 * h + t) + j : (t == 12 ? 120 + 4 * h + j : 5 * (12 * h + 4 * (t - 13) + j) + 4);
}

// ---------------------------------------------------------------------------
// Activation prep: four waves per (row, 1024-chunk), wave w on quarter w.
//   input  = x (times the row's RMS scale when rms_eps > 0 and the per-channel
//            gain when given), or silu(g) * u
//   value  = bf16_rne((1/32) H (signs * input))   (rotation when signs given)
// Output: MFMA A fragments.  For 32-row group mt, block kb, step s (0..7)
// and lane l the 16 bytes at element offset (((mt nb + kb) 8 + s) 64 + l) 8
// hold A[32 mt + l % 32][128 kb + gemm_kperm(8 f + j)], j = 0..7, with
// f = s (l < 32) or gemm_hi_frag(s) (l >= 32) -- the operand of
// v_mfma_f32_32x32x16_bf16 for that step.
// Rows >= m are never written: an output row of the MFMA depends only on
// its own A row, so whatever they hold only reaches outputs nobody stores.
// Q2 (the PQ2_0 GEMM): fragment f = 8 h + s holds weights 8 f .. 8 f + 7 in
// order, i.e. step s, half h takes block positions 64 h + 8 s + j, which are
// the two code bytes 16 h + 2 s, 16 h + 2 s + 1 of a PQ2_0 block.
// ---------------------------------------------------------------------------
// W8: 8-bit activations instead (x given, no rotation, no norm): the row's
// max |x| comes from the same whole-row loads as the mean square, the chunk
// becomes q = rint(x * float(127 / max|x|)) and is written as int8 operands
// of v_mfma_i32_32x32x32_i8: for 32-row group mt, block kb, step s (0..3)
// and lane l the 16 bytes at byte offset (((mt nb + kb) 4 + s) 64 + l) 16
// hold q[32 mt + l % 32][128 kb + gemm_i8_kperm(32 s + 16 (l / 32) + i)],
// i = 0..15; wave 0 of the row also stores its step max|x| / 127.
// Workgroup of the stream-K range holding unit u: the largest w with
// floor(w U / G) <= u, that is with w U < (u + 1) G.
__device__ __forceinline__ int64_t gemm_owner(int64_t u, int64_t units, int64_t G)
{
    return ((u + 1) * G + units - 1) / units - 1;
}

// The gate+up outputs read by the down projection's prep when the gate+up
// GEMM's fix-up has not run: whole tiles, and shared tiles one workgroup
// covered, are final in y; any other shared tile is the sum of its partials
// in workgroup order, added exactly as k_gemm_fix adds them and stored back
// to y.  The prep takes this path only when no shared tile has more than
// kSkPre workgroups (gemm_fold_ok), so every partial is requested up front.
constexpr int kSkPre = 4;

struct SkRead {
    gm_f32x4 y, p[kSkPre];
    int64_t w_lo, w_hi;
};

__device__ __forceinline__ void sk_issue(const SkView &v, const float *yp, int64_t row, int64_t vc, SkRead &s)
{
    s.y = *reinterpret_cast<const gm_f32x4 *>(yp);
    const int64_t tm = row / v.prow, r = row - tm * v.prow;
    const int64_t t = (vc / kGemmBN) * v.tiles_m + tm;
    s.w_lo = 0;
    s.w_hi = 0;
    int64_t k_lo = 0;
    if (t >= v.dp_tiles) {
        const int64_t first_u = (t - v.dp_tiles) * v.nb;
        s.w_lo = gemm_owner(first_u, v.sk_units, v.sk_wgs);
        s.w_hi = gemm_owner(first_u + v.nb - 1, v.sk_units, v.sk_wgs);
        k_lo = (s.w_lo * v.sk_units < first_u * v.sk_wgs) ? 1 : 0;
    }
    if (s.w_lo < s.w_hi) {
        // w_lo's segment of this tile is its first partial unless its range
        // began in an earlier tile; every later workgroup's is its first
        const int64_t seg = 2 * v.prow * kGemmBN;
        const float *p0 = v.part + r * kGemmBN + (vc % kGemmBN);
#pragma unroll
        for (int i = 0; i < kSkPre; ++i) {
            const int64_t w = s.w_lo + i <= s.w_hi ? s.w_lo + i : s.w_hi;  // clamped: no branch
            s.p[i] = *reinterpret_cast<const gm_f32x4 *>(p0 + w * seg + (i == 0 ? k_lo * v.prow * kGemmBN : 0));
        }
    }
}

__device__ __forceinline__ gm_f32x4 sk_finish(const SkRead &s, float *yp)
{
    if (s.w_lo == s.w_hi) return s.y;
    gm_f32x4 acc = s.p[0];
#pragma unroll
    for (int i = 1; i < kSkPre; ++i)
        if (s.w_lo + i <= s.w_hi) acc += s.p[i];
    *reinterpret_cast<gm_f32x4 *>(yp) = acc;
    return acc;
}

constexpr int kPrepThreads = 4 * kWave;

template <bool Q2, bool W8>
__global__ void __launch_bounds__(kPrepThreads) k_prep_frag(
    const float *__restrict__ x, const float *g, const float *u,  // g, u: completed in place on the stream-K path
    int64_t k, const float *__restrict__ signs, float rms_eps, const float *__restrict__ gain,
    uint16_t *__restrict__ xf, float *__restrict__ step, SkView sk)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ f32x4 qt[kPrepThreads];  // the four quarters' 256-point transforms
    __shared__ float st[kHadamard];     // the finished chunk in natural order
    __shared__ float red[kPrepThreads / kWave];
    const int64_t cpr = (k + kHadamard - 1) / kHadamard;  // == k / 1024 when signs are given
    const int64_t row = blockIdx.x / cpr;
    const int64_t ch = blockIdx.x - row * cpr;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;                     // quarter of the chunk
    const int ec = (kHadamard / 4) * w + 4 * lane;  // this thread's four elements of the chunk
    const int64_t e = ch * kHadamard + ec;         // ... of the row
    const int64_t ecl = e < k ? e : k - 4;         // k is a multiple of 128: e < k covers all four
    // Every load is requested before any arithmetic (clamped addresses, no
    // branches around the loads but workgroup-uniform ones): the four values
    // of x or of g and u, the gain, the signs and this thread's share of the
    // row for its mean square or max.  Requested one after another's use,
    // they cost a dependent round trip to memory each.
    constexpr int kQ = 6;  // 16-byte loads of the row per thread per batch (one batch for k <= 6144)
    const float *src0 = x != nullptr ? x : g;
    const bool rms = !W8 && x != nullptr && rms_eps > 0.0f;
    const f32x4 *xr = reinterpret_cast<const f32x4 *>(src0 + row * k);
    const int64_t k4 = k / 4;
    // g and u through the gate+up GEMM's stream-K partials (sk.part set,
    // x == nullptr): the g columns are the virtual matrix's first k, u's the next k
    const bool skv = x == nullptr && sk.part != nullptr;  // kernel-uniform
    SkRead skg, sku;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 uw = {1.0f, 1.0f, 1.0f, 1.0f};
    if (skv) {
        sk_issue(sk, g + row * k + ecl, row, ecl, skg);
        sk_issue(sk, u + row * k + ecl, row, k + ecl, sku);
    } else {
        v = *reinterpret_cast<const f32x4 *>(src0 + row * k + ecl);
        if (x == nullptr)
            uw = *reinterpret_cast<const f32x4 *>(u + row * k + ecl);
        else if (gain != nullptr)  // the norm's per-channel weight (uw holds it on this path)
            uw = *reinterpret_cast<const f32x4 *>(gain + ecl);
    }
    f32x4 sg = {1.0f, 1.0f, 1.0f, 1.0f};
    if (signs != nullptr) sg = *reinterpret_cast<const f32x4 *>(signs + ec);
    f32x4 xv[kQ];
    if (rms || W8) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int64_t i = tid + static_cast<int64_t>(kPrepThreads) * q;
            xv[q] = xr[i < k4 ? i : k4 - 1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (skv && e < k) {  // e < k always here (k is a multiple of 1024 on this path)
        v = sk_finish(skg, const_cast<float *>(g) + row * k + ecl);
        uw = sk_finish(sku, const_cast<float *>(u) + row * k + ecl);
    }
    if (x == nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = v[j] / (1.0f + expf(-v[j])) * uw[j];
    } else if (gain != nullptr) {
        v *= uw;
    }
    if (e >= k) v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // this wave's part of the row's sum of squares (or of its max |x|),
    // batch by batch (the first one requested above; clamped copies repeat
    // a real element, so they are masked for the sum and harmless for the max)
    if (rms) {
        float sq = 0.0f;
        for (int64_t i0 = 0; i0 < k4; i0 += static_cast<int64_t>(kQ) * kPrepThreads) {
            if (i0 > 0) {
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const int64_t i = i0 + tid + static_cast<int64_t>(kPrepThreads) * q;
                    xv[q] = xr[i < k4 ? i : k4 - 1];
                }
            }
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                const float m = i0 + tid + static_cast<int64_t>(kPrepThreads) * q < k4 ? 1.0f : 0.0f;
                sq = fmaf(m * xv[q].x, xv[q].x, fmaf(m * xv[q].y, xv[q].y, fmaf(m * xv[q].z, xv[q].z,
                                                                                 fmaf(m * xv[q].w, xv[q].w, sq))));
            }
        }
        sq = wave_sum(sq);
        if (lane == 0) red[w] = sq;
    }
    if constexpr (W8) {
        float mx = 0.0f;
        for (int64_t i0 = 0; i0 < k4; i0 += static_cast<int64_t>(kQ) * kPrepThreads) {
            if (i0 > 0) {
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const int64_t i = i0 + tid + static_cast<int64_t>(kPrepThreads) * q;
                    xv[q] = xr[i < k4 ? i : k4 - 1];
                }
            }
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[q].x), fabsf(xv[q].y)), fmaxf(fabsf(xv[q].z), fabsf(xv[q].w))));
        }
        mx = wave_max(mx);
        if (lane == 0) red[w] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float c = mx > 0.0f ? static_cast<float>(127.0 / static_cast<double>(mx)) : 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = rintf(v[j] * c);
        if (ch == 0 && tid == 0) step[row] = static_cast<float>(static_cast<double>(mx) / 127.0);
        *reinterpret_cast<f32x4 *>(st + ec) = v;
    } else if (signs != nullptr) {
        // R = (1/32) H_1024 D_s with H_1024 = H_4 (x) H_256 (the top two index
        // bits the H_4 factor): each wave transforms its quarter, and output
        // quarter w = sum_c (-1)^popcount(w & c) H_256 quarter c
        float t4[4] = {v[0] * sg[0], v[1] * sg[1], v[2] * sg[2], v[3] * sg[3]};
        fwht256_wave(t4);
        qt[tid] = f32x4{t4[0], t4[1], t4[2], t4[3]};
        __syncthreads();
        const float a = rms ? 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / static_cast<float>(k) + rms_eps)
                            : 1.0f;
        const f32x4 q0 = qt[lane], q1 = qt[kWave + lane], q2 = qt[2 * kWave + lane], q3 = qt[3 * kWave + lane];
        const float s1 = (w & 1) ? -1.0f : 1.0f, s2 = (w & 2) ? -1.0f : 1.0f;  // row w of H_4
        const f32x4 t = (q0 + s1 * q1) + s2 * (q2 + s1 * q3);
        *reinterpret_cast<f32x4 *>(st + ec) = t * ((1.0f / 32.0f) * a);
    } else {
        if (rms) {
            __syncthreads();
            v *= 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / static_cast<float>(k) + rms_eps);
        }
        *reinterpret_cast<f32x4 *>(st + ec) = v;
    }
    __syncthreads();

    const int64_t nb = k / kBlockWeights;
    const int64_t mt = row / 32;
    const int rl = static_cast<int>(row % 32);
    if constexpr (W8) {
        // one piece per thread of wave 0: block kbl of the chunk, step stp, half h
        if (tid >= kWave) return;
        const int kbl = tid >> 3, stp = (tid >> 1) & 3, h = tid & 1;
        const int64_t kb = ch * (kHadamard / kBlockWeights) + kbl;
        if (kb < nb) {
            const float *src = st + kBlockWeights * kbl;
            gm_u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t d = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int32_t qi = static_cast<int32_t>(src[gemm_i8_kperm(32 * stp + 16 * h + 4 * q + j)]);
                    d |= (static_cast<uint32_t>(qi) & 0xffu) << (8 * j);
                }
                o[q] = d;
            }
            uint8_t *xq = reinterpret_cast<uint8_t *>(xf);
            *reinterpret_cast<gm_u32x4 *>(xq + (((mt * nb + kb) * 4 + stp) * kWave + rl + 32 * h) * 16) = o;
        }
        return;
    }
    // one fragment piece per thread of waves 0 and 1: block kbl of the chunk, fragment f
    if (tid >= 2 * kWave) return;
    {
        const int p = tid;
        const int kbl = p >> 4, f = p & 15;
        const int64_t kb = ch * (kHadamard / kBlockWeights) + kbl;
        if (kb >= nb) return;
        const float *src = st + kBlockWeights * kbl;
        gm_u32x4 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int w0 = Q2 ? 8 * f + 2 * jj : gemm_kperm(8 * f + 2 * jj);
            const int w1 = Q2 ? 8 * f + 2 * jj + 1 : gemm_kperm(8 * f + 2 * jj + 1);
            const uint32_t lo = f32_to_bf16_rne(src[w0]);
            const uint32_t hi = f32_to_bf16_rne(src[w1]);
            o[jj] = lo | (hi << 16);
        }
        // (step, half) that carries fragment f
        const int fs = Q2 ? (f & 7) : (f < 8 ? f : (f < 10 ? f - 3 : (f < 15 ? f - 10 : 7)));
        const int fh = f < 8 ? 0 : 1;
        const int64_t off = (((mt * nb + kb) * 8 + fs) * kWave + rl + 32 * fh) * 8;
        *reinterpret_cast<gm_u32x4 *>(xf + off) = o;
    }
}

// ---------------------------------------------------------------------------
// MFMA GEMM.  A workgroup (4 or 8 waves) owns 128 output columns (weight
// rows) and BM = 32 TM WM output rows; the waves form a WM x WN grid, each
// owning TM x TN 32x32 tiles of v_mfma_f32_32x32x16_bf16.  K advances one
// PTQ1_0 block per iteration:
//   B: every thread decodes part of one column's 28-byte block through a
//      byte -> 5 trits table into LDS fragments.  Three buffers rotate:
//      while block i is multiplied, block i + 2 is decoded and the first
//      fragments of block i + 1 are already being read, so the MFMA
//      pipeline runs on across the one barrier per block;
//   A: each wave loads its 16-byte activation fragments from global memory
//      a few MFMA steps ahead;
//   8 MFMA steps accumulate the block's partial product from zero, then
//      acc += partial * scale[column] in fp32.
// Trits are stored as bf16 -2 / 0 / +2 (low byte always zero, so a table
// entry is just the five high bytes) and the scale is halved to match.
// Work split: the grid fills the CUs once; each workgroup takes whole tiles
// for as many full rounds as there are, then (stream-K) an equal run of the
// remaining tiles' (tile, K block) units in tile order, as one segment per
// tile it touches.  A segment covering all blocks of its tile stores the
// result; any other stores an fp32 partial, and k_gemm_fix adds the
// partials of each shared tile in workgroup order.
// Operand layouts (gfx950, 32x32x16 bf16): lane l supplies A[l%32][8(l/32)+j]
// and B[8(l/32)+j][l%32], j = 0..7; result register r of lane l is
// D[8(r/4) + 4(l/32) + r%4][l%32].
//
// LDS (160 KB): [0, 64 KB) holds 256 rows of 256 bytes, row b for byte
// value b: 16 copies of its 8-byte table entry in the first half (lane l
// reads copy l % 16), and in the second half of rows 0..11 the block
// scales [buffer][column]; [64 KB, 160 KB) holds the three decoded blocks.
// ---------------------------------------------------------------------------
constexpr int kFragsPerBlock = 16;                             // per column, 16 B each
constexpr int kBufBytes = kFragsPerBlock * kGemmBN * 16;        // 32 KB per decoded block
constexpr int kNumBufs = 3;
constexpr int kTabCopies = 16;
constexpr int kTabBytes = 256 * 256;
constexpr int kGemmLds = kTabBytes + kNumBufs * kBufBytes;
static_assert(kGemmLds <= 160 * 1024, "LDS");
static_assert(kNumBufs * kGemmBN <= 12 * 32, "scales fit in the free halves of rows 0..11");

// LDS byte offset of the scale of (buffer, column)
__device__ __forceinline__ uint32_t gemm_scale_addr(int buf, int col)
{
    const uint32_t i = static_cast<uint32_t>(buf * kGemmBN + col);
    return (i >> 5) * 256u + 128u + (i & 31u) * 4u;
}

// bf16 high byte of 2 * (digit - 1): digit 0 -> -2 (0xC0), 1 -> 0, 2 -> +2 (0x40)
__device__ __forceinline__ uint32_t trit_hi(uint32_t d) { return d == 0 ? 0xC0u : (d == 1 ? 0x00u : 0x40u); }

// v_perm selector: fragment dword of digit d for bytes (x, y) taken from the
// table entries' dword (d < 4 ? 0 : 1): [0, H_d(x), 0, H_d(y)].
__device__ __forceinline__ constexpr uint32_t dsel(int d)
{
    return 0x000c000cu | (static_cast<uint32_t>(d & 3) << 8) | (static_cast<uint32_t>(4 + (d & 3)) << 24);
}

struct GemmArgs {
    const uint16_t *xf;      // A fragments (k_prep_frag layout)
    const uint8_t *w0;       // tiled matrix 0 (rows [0, n0) of the virtual matrix)
    const uint8_t *w1;       // tiled matrix 1 (rows [n0, n0 + n1)), may be null
    int64_t n0, n1, bands0, bands1;
    float *y0, *y1;          // outputs [m][n0], [m][n1]
    const float *residual;   // [m][n0] or null
    float *part;             // partial tiles [workgroup][first / last][prow][128]
    const float *row_scale;  // int8 path: each output row times row_scale[row] (the W2A8 step)
    int64_t m, nb;           // activation rows, K blocks
    int64_t tiles_m, prow;   // row tiles; rows of a row tile (= m with one row tile)
    int64_t wgs;             // workgroups
    int64_t dp_rounds;       // rounds of whole tiles per workgroup (tiles [0, dp_tiles))
    int64_t dp_tiles;        // dp_rounds x wgs
    int64_t sk_units;        // (tiles - dp_tiles) x K blocks, shared evenly by
    int64_t sk_wgs;          // workgroups [0, sk_wgs), sk_wgs = min(wgs, sk_units)
};

template <int WM, int WN, int TM, int TN, int PD>
__global__ void __launch_bounds__(64 * WM * WN) k_gemm_mfma(GemmArgs a)
{
    constexpr int kNT = 64 * WM * WN;  // 256 or 512 threads
    static_assert((kNT == 256 || kNT == 512) && WN * TN * 32 == kGemmBN, "4 or 8 waves x 128 columns");
    static_assert(PD % kNumBufs == 0, "weight ring: a multiple of the B buffers");
    constexpr int kBq = 1;  // B-fragment prefetch, MFMA steps (ring of 2)
    constexpr int kAr = 4;  // activation-fragment ring, MFMA steps
    // step s of every block uses ring slots s % (kBq + 1) and s % kAr: both
    // rings must divide the block's eight steps so every block starts at slot 0
    static_assert(8 % (kBq + 1) == 0 && 8 % kAr == 0, "rings divide the eight MFMA steps of a block");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *tab = lds;
    char *bsm = lds + kTabBytes;
    typedef __attribute__((address_space(3))) float lds_f32;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t rows = a.n0 + a.n1;

    // ---- byte -> trit table: entry b, copy c at b * 256 + c * 8
    {
        const uint32_t b = static_cast<uint32_t>(tid & 255);
        uint32_t r = b, h[5];
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            const uint32_t t = 3u * r;
            h[n] = trit_hi(t >> 8);
            r = t & 0xffu;
        }
        const gm_u32x2 e = {h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24), h[4]};
        constexpr int kCopiesPerThread = kTabCopies * 256 / kNT;
        const int c0 = (tid >> 8) * kCopiesPerThread;
#pragma unroll
        for (int i = 0; i < kCopiesPerThread; ++i)
            *reinterpret_cast<gm_u32x2 *>(tab + b * 256 + ((b + c0 + i) & (kTabCopies - 1)) * 8) = e;
    }

    // ---- work split: whole tiles wg, wg + G, ... for the first dp_rounds
    // rounds, then units [w U / G, (w + 1) U / G) of the U = (remaining
    // tiles) x blocks, one segment per tile touched (tile t = column tile
    // t / tiles_m, row tile t % tiles_m).
    const int64_t G = gridDim.x, wg = blockIdx.x;
    const int64_t Gs = a.sk_wgs;  // workgroups [0, Gs) share the stream-K units
    const int64_t sk_lo = wg < Gs ? wg * a.sk_units / Gs : 0, sk_hi = wg < Gs ? (wg + 1) * a.sk_units / Gs : 0;
    int64_t jdp = 0, useg = sk_lo;
    while (jdp < a.dp_rounds || useg < sk_hi) {
        int64_t tile, kb0;
        int nblk, kslot = 0;
        bool full;
        if (jdp < a.dp_rounds) {  // whole tile wg + jdp G
            tile = wg + jdp * G;
            kb0 = 0;
            nblk = static_cast<int>(a.nb);
            full = true;
            ++jdp;
        } else {  // units [useg, uend) of stream-K tile t2
            const int64_t t2 = useg / a.nb;
            kb0 = useg - t2 * a.nb;
            const int64_t uend = (t2 + 1) * a.nb < sk_hi ? (t2 + 1) * a.nb : sk_hi;
            nblk = static_cast<int>(uend - useg);
            tile = a.dp_tiles + t2;
            full = kb0 == 0 && nblk == a.nb;
            kslot = useg == sk_lo ? 0 : 1;
            useg = uend;
        }
        const int last = nblk - 1;
        auto blk = [&](int i) -> int64_t { return kb0 + (i < last ? i : last); };  // clamped block index
        const int64_t tn = tile / a.tiles_m, tm = tile - tn * a.tiles_m;
        const int64_t tile_n = tn * kGemmBN;
        const int64_t mt0 = (tm * WM + wm) * TM;  // this wave's first 32-row group
        const bool active = mt0 * 32 < a.m;

        // ---- this thread's share of the decode: column dn and a byte range of
        //      its block.  256 threads: bytes [0,12) (role 0) or [12,28) (role 1);
        //      512 threads: bytes [0,8), [8,16), [16,24) (roles 0-2, five whole
        //      fragments each) or [20,28) (role 3: fragment 15 and the scale).
        const int dn = tid & (kGemmBN - 1);
        const int role = tid >> 7;
        const int64_t gcol = tile_n + dn;
        const uint8_t *wcol = a.w0;
        int64_t sstride = 0;
        if (gcol < rows) {
            const bool first = gcol < a.n0;
            const int64_t rr = first ? gcol : gcol - a.n0;
            wcol = (first ? a.w0 : a.w1) + (rr / kTileRows) * kTileBytes + (rr % kTileRows) * (kTileBlocks * kBlockBytes);
            sstride = (first ? a.bands0 : a.bands1) * kTileBytes;
        }
        wcol += kNT == 256 ? role * 12 : (role < 3 ? 8 * role : 20);
        const uint32_t lc = static_cast<uint32_t>(lane & (kTabCopies - 1)) << 3;

        // Loads are unconditional (callers clamp the block) so that the
        // compiler's in-order load counting never has to merge two paths.
        auto load_w = [&](gm_u32x4 &r, int64_t kb) {  // 256 threads: role 0 uses 3 of the 4 dwords
            const uint8_t *p = wcol + (kb >> 1) * sstride + (kb & 1) * kBlockBytes;
            if constexpr (kNT == 256) {
                r = *reinterpret_cast<const gm_u32x4a *>(p);
            } else {
                const gm_u32x2a v = *reinterpret_cast<const gm_u32x2a *>(p);
                r = gm_u32x4{v[0], v[1], 0u, 0u};
            }
        };
        // The table sits at LDS address 0 (the kernel has no static LDS), so the
        // v_perm result is the complete LDS address.
        typedef __attribute__((address_space(3))) const gm_u32x2 lds_u32x2;
        auto tab_read = [&](uint32_t w, int byte) -> gm_u32x2 {
            const uint32_t addr = __builtin_amdgcn_perm(lc, w, 0x0c0c0004u | (static_cast<uint32_t>(byte) << 8));
            return *reinterpret_cast<lds_u32x2 *>(static_cast<uintptr_t>(addr));
        };
        // 256 threads, both roles in one branch-free sequence over their bytes:
        //   an 8-byte group  -> 5 whole fragments (role 0: bytes 0-7 -> fragments
        //                       0-4; role 1: bytes 16-23 -> fragments 10-14),
        //   a 4-byte half    -> half of fragments 5-9 (role 0: bytes 8-11, low
        //                       8 bytes; role 1: bytes 12-15, high 8 bytes),
        //   fragment 15 and the scale from bytes 24-27 (role 1 only).
        const int grp_frag = role ? 10 : 0;
        const int half_off = role ? 8 : 0;
        struct TabRegs {
            gm_u32x2 tg[8], th[4], tt[2];
            uint32_t tw;
        };
        auto decode_read = [&](const gm_u32x4 &r, TabRegs &q, int part_no) {
            if constexpr (kNT == 512) {
                if (part_no == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) q.tg[i] = tab_read(r[0], i);
#pragma unroll
                    for (int i = 0; i < 4; ++i) q.tg[4 + i] = tab_read(r[1], i);
                    q.tw = r[1];
                }
            } else if (part_no == 0) {
                const uint32_t g0 = role ? r[1] : r[0], g1 = role ? r[2] : r[1];
#pragma unroll
                for (int i = 0; i < 4; ++i) q.tg[i] = tab_read(g0, i);
#pragma unroll
                for (int i = 0; i < 4; ++i) q.tg[4 + i] = tab_read(g1, i);
            } else {
                const uint32_t hw = role ? r[0] : r[2];
                q.tw = r[3];
#pragma unroll
                for (int i = 0; i < 4; ++i) q.th[i] = tab_read(hw, i);
                q.tt[0] = tab_read(q.tw, 0);
                q.tt[1] = tab_read(q.tw, 1);
            }
        };
        // fragment fifteen from the table entries of bytes 24 and 25
        auto frag15 = [&](gm_u32x2 t24, gm_u32x2 t25) -> gm_u32x4 {
            return gm_u32x4{__builtin_amdgcn_perm(t24[0], t24[0], 0x010c000cu),
                            __builtin_amdgcn_perm(t24[0], t24[0], 0x030c020cu),
                            __builtin_amdgcn_perm(t25[0], t24[1], 0x040c000cu),
                            __builtin_amdgcn_perm(t25[0], t25[0], 0x020c010cu)};
        };
        auto put_scale = [&](int buf, uint32_t tw) {
            *reinterpret_cast<lds_f32 *>(static_cast<uintptr_t>(gemm_scale_addr(buf, dn))) =
                0.5f * half_bits_to_float(tw >> 16);
        };
        // fragment group d (0..4) of the decoded block, or (d == 5) fragment 15
        // and the scale
        auto decode_write = [&](const TabRegs &q, int buf, int d) {
            char *bw = bsm + buf * kBufBytes;
            if constexpr (kNT == 512) {
                if (d >= 5) return;
                if (role < 3) {  // wave-uniform
                    const int c = d >> 2;
                    const gm_u32x4 o = {__builtin_amdgcn_perm(q.tg[1][c], q.tg[0][c], dsel(d)),
                                        __builtin_amdgcn_perm(q.tg[3][c], q.tg[2][c], dsel(d)),
                                        __builtin_amdgcn_perm(q.tg[5][c], q.tg[4][c], dsel(d)),
                                        __builtin_amdgcn_perm(q.tg[7][c], q.tg[6][c], dsel(d))};
                    *reinterpret_cast<gm_u32x4 *>(bw + ((5 * role + d) * kGemmBN + dn) * 16) = o;
                } else if (d == 0) {  // bytes 20..27: 24 and 25 are entries 4 and 5
                    *reinterpret_cast<gm_u32x4 *>(bw + (15 * kGemmBN + dn) * 16) = frag15(q.tg[4], q.tg[5]);
                    put_scale(buf, q.tw);
                }
            } else if (d < 5) {
                const int c = d >> 2;
                const gm_u32x4 o = {__builtin_amdgcn_perm(q.tg[1][c], q.tg[0][c], dsel(d)),
                                    __builtin_amdgcn_perm(q.tg[3][c], q.tg[2][c], dsel(d)),
                                    __builtin_amdgcn_perm(q.tg[5][c], q.tg[4][c], dsel(d)),
                                    __builtin_amdgcn_perm(q.tg[7][c], q.tg[6][c], dsel(d))};
                *reinterpret_cast<gm_u32x4 *>(bw + ((grp_frag + d) * kGemmBN + dn) * 16) = o;
                const gm_u32x2 h = {__builtin_amdgcn_perm(q.th[1][c], q.th[0][c], dsel(d)),
                                    __builtin_amdgcn_perm(q.th[3][c], q.th[2][c], dsel(d))};
                *reinterpret_cast<gm_u32x2 *>(bw + ((5 + d) * kGemmBN + dn) * 16 + half_off) = h;
            } else if (role == 1) {  // wave-uniform
                *reinterpret_cast<gm_u32x4 *>(bw + (15 * kGemmBN + dn) * 16) = frag15(q.tt[0], q.tt[1]);
                put_scale(buf, q.tw);
            }
        };
        auto decode_all = [&](const gm_u32x4 &r, int buf) {
            TabRegs q;
            decode_read(r, q, 0);
            decode_read(r, q, 1);
#pragma unroll
            for (int d = 0; d < 6; ++d) decode_write(q, buf, d);
        };

        // activation fragments: this wave's 32-row groups mt0 .. mt0 + TM - 1
        const uint16_t *xw = a.xf + (mt0 * a.nb * 8 * kWave + lane) * 8;
        const int64_t tm_stride = a.nb * 8 * kWave * 8;
        auto load_a = [&](gm_u32x4 (&f)[TM], int64_t kb, int s) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
                f[m] = *reinterpret_cast<const gm_u32x4 *>(xw + m * tm_stride + (kb * 8 + s) * kWave * 8);
        };

        f32x16 acc[TM][TN], part[TM][TN];
        float scl[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            scl[t] = 0.0f;
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][t][r] = part[m][t][r] = 0.0f;
        }
        const int scol = wn * 32 * TN + (lane & 31);
        // B fragment of step s: fragment s (lanes 0-31) or gemm_hi_frag(s)
        // (lanes 32-63); the difference takes three values, folded into three
        // per-lane bases
        const int hi = lane >> 5;
        const char *bsr0 = bsm + scol * 16 + hi * (10 * kGemmBN * 16);
        const char *bsr1 = bsm + scol * 16 + hi * (3 * kGemmBN * 16);
        const char *bsr2 = bsm + scol * 16 + hi * (8 * kGemmBN * 16);
        auto read_b = [&](bf16x8 (&dst)[TN], int buf, int step) {
            const char *b = step < 5 ? bsr0 : (step < 7 ? bsr1 : bsr2);
#pragma unroll
            for (int t = 0; t < TN; ++t)
                dst[t] = *reinterpret_cast<const bf16x8 *>(b + buf * kBufBytes + (step * kGemmBN + 32 * t) * 16);
        };

        // ---- prologue: blocks 0 and 1 decoded, block 2 .. of weights, the first
        //      activation steps and the first B fragments in flight
        gm_u32x4 afr[kAr][TM];
        bf16x8 bq[kBq + 1][TN];
        gm_u32x4 ring[PD];  // weights of blocks i + 2 .. i + 1 + PD at iteration i
        {
            gm_u32x4 w_first, w_second;
            load_w(w_first, blk(0));
            load_w(w_second, blk(1));
#pragma unroll
            for (int p = 0; p < PD; ++p) load_w(ring[(2 + p) % PD], blk(2 + p));
#pragma unroll
            for (int s = 0; s < kAr; ++s) load_a(afr[s], blk(0), s);
            __syncthreads();  // table
            decode_all(w_first, 0);
            decode_all(w_second, 1);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kBq; ++p) read_b(bq[p], 0, p);

        // One block of K, as eight MFMA steps.  Each step also carries part of
        // the surrounding work, in a fixed order (sched_barrier keeps it): the
        // B fragments kBq steps ahead (into the next block's buffer at the end),
        // the activation fragments kAr steps ahead and a slice of the decode of
        // block i + 2 (table reads in steps 0-1, fragment groups in steps 2-7).
        // Step 0 first folds the previous block's partial into acc (acc += part
        // * scale), tile by tile, just before that tile's MFMA chain restarts.
        auto iteration = [&](int buf, int i, gm_u32x4 &rslot) {
            const int nbuf = (buf + 1) % kNumBufs, dbuf = (buf + 2) % kNumBufs;
            TabRegs q;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                if (s + kBq < 8)
                    read_b(bq[(s + kBq) % (kBq + 1)], buf, s + kBq);
                else
                    read_b(bq[(s + kBq) % (kBq + 1)], nbuf, s + kBq - 8);
                {
                    gm_u32x4 (&ar)[TM] = afr[s % kAr];
                    bf16x8 av[TM];
#pragma unroll
                    for (int m = 0; m < TM; ++m) av[m] = __builtin_bit_cast(bf16x8, ar[m]);
#pragma unroll
                    for (int m = 0; m < TM; ++m)
#pragma unroll
                        for (int t = 0; t < TN; ++t) {
                            if (s == 0) {
#pragma unroll
                                for (int r = 0; r < 16; ++r) acc[m][t][r] = fmaf(part[m][t][r], scl[t], acc[m][t][r]);
                                const f32x16 z = {};
                                part[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bq[0][t], z, 0, 0, 0);
                            } else {
                                part[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bq[s % (kBq + 1)][t],
                                                                                      part[m][t], 0, 0, 0);
                            }
                        }
                    if (s + kAr < 8)
                        load_a(ar, blk(i), s + kAr);
                    else
                        load_a(ar, blk(i + 1), s + kAr - 8);
                }
                if (s < 2) {
                    decode_read(rslot, q, s);
                    if (s == 1) load_w(rslot, blk(i + 2 + PD));
                } else {
                    decode_write(q, dbuf, s - 2);
                }
                if (s == 7) {
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        scl[t] = *reinterpret_cast<const lds_f32 *>(
                            static_cast<uintptr_t>(gemm_scale_addr(buf, scol + 32 * t)));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        for (int base = 0; base < nblk; base += PD) {
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                const int i = base + u;
                if (i >= nblk) break;
                iteration(u % kNumBufs, i, ring[(u + 2) % PD]);
                __syncthreads();
            }
        }
        // the last block's partial is not scaled yet
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][t][r] = fmaf(part[m][t][r], scl[t], acc[m][t][r]);

        // a segment over all blocks of its tile is final; any other is stored
        // as this workgroup's first (0) or last (1) partial for k_gemm_fix
        float *pp = a.part + (wg * 2 + kslot) * a.prow * kGemmBN;
        const int64_t row0 = tm * a.prow;  // first row of the tile
        // the row offsets below are the same in every segment; an opaque lane
        // index keeps the compiler from hoisting them out of the segment loop
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        if (active) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    const int64_t col = tile_n + wn * 32 * TN + 32 * t + (lane_e & 31);
                    if (col >= rows) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t row = (mt0 + m) * 32 + 8 * (r / 4) + 4 * (lane_e / 32) + (r % 4);
                        if (row >= a.m) continue;
                        const float v = acc[m][t][r];
                        if (!full) {
                            pp[(row - row0) * kGemmBN + (col - tile_n)] = v;
                        } else if (col < a.n0) {
                            const int64_t o = row * a.n0 + col;
                            a.y0[o] = a.residual ? a.residual[o] + v : v;
                        } else {
                            a.y1[row * a.n1 + (col - a.n0)] = v;
                        }
                    }
                }
        }
    }  // segments
}


// ---------------------------------------------------------------------------
// Small-batch GEMM (M <= 64): every wave decodes the B fragments of its own
// 32 columns straight into registers, so no decoded block goes through LDS;
// the byte -> trit table (read-only after its build) sits in LDS, and two
// workgroups share a CU.  Up to 16 rows, the block's activation fragments
// are staged in LDS as well (below), with one barrier per block; above, the
// loop has no barrier and every wave loads its activation fragments.
//
// A workgroup (4 waves) owns 128 columns and 32 TM rows; wave w owns columns
// 32 w .. 32 w + 31, all TM row groups.  Lane l (column l % 32, half
// h = l / 32) loads 16 bytes of its column's block at byte 8 h and the dword
// at byte 24 (the scale, and bytes 24-25 for lanes 32-63), looks up the 18
// table entries it needs and builds, for MFMA step s, the fragment of the
// step/half mapping above: steps 0-4 take digit s of its first 8 bytes
// (bytes 0-7 in lanes 0-31, 16-23 in lanes 32-63), steps 5-7 digits of
// bytes 8-15 (0, 1, 2 in lanes 0-31; 3, 4 and fragment 15 in lanes 32-63).
// Table entries here are [H0 H1 H2 H3 | H4 H1 H2 H3] so that the two halves'
// digits of steps 5 and 6 sit in the same dword.
//
// Q2: the same kernel over a PQ2_0 tiled matrix ("Why I Am Building Another
// Inference Engine", Level 2).  A table entry is the four weights of a code
// byte as bf16 (-1, 0, +1; code 3 -> 0), low field first, so the fragment of
// step s is the entries of code bytes 16 h + 2 s and 16 h + 2 s + 1 side by
// side (activations in the prep kernel's Q2 order).  Lane l loads the 16
// code bytes 16 h .. 16 h + 15 of its column's block and the tile's dword
// of that row's two scales; the scale is applied unhalved.
// ---------------------------------------------------------------------------
constexpr int kRdThreads = 256;
constexpr int kRdTabCopies = 32;                    // conflict-free 8-byte reads
constexpr int kRdLds = 256 * kRdTabCopies * 8;      // 64 KB: two workgroups per CU

// Small batches (one 32-row tile, at most 16 live rows): the activation
// fragments of a block are loaded once per workgroup into LDS (one 16-byte
// piece per live (step, half, row), read by all four waves) instead of by
// every wave from global memory, which cuts the address unit's work per
// block from 40 load instructions to 10 (batch 8: the 34816 x 5120 GEMM
// 15.4 -> 14.4 us, the FFN block 49.5 -> 46 us).  Two slots alternate by
// block: block i + 1's pieces (loaded one block earlier) are written at the
// start of block i, and a barrier halfway through block i, before the
// fragments of block i + 1 are read, orders both the writes and the last
// reads of that slot (block i - 1's).
__host__ __device__ constexpr bool rd_lds_a(int TM, int LR) { return TM == 1 && LR <= 2; }
__host__ __device__ constexpr int rd_a_slot(int LR) { return 8 * 2 * 8 * LR * 16; }  // bytes per block

// v_perm selector: [0, byte b of x's entry, 0, byte b of y's entry]
__device__ __forceinline__ constexpr uint32_t rd_sel(int b)
{
    return 0x000c000cu | (static_cast<uint32_t>(b) << 8) | (static_cast<uint32_t>(4 + b) << 24);
}

// LR: 8-row groups of the last row tile that hold activation rows (the
// others are zero padding and are neither scaled nor stored).
template <int TM, int PD, int LR, bool Q2>
__global__ void __launch_bounds__(kRdThreads, 2) k_gemm_rd(GemmArgs a)
{
    static_assert(LR >= 1 && LR <= 4, "8-row groups of a 32-row tile");
    static_assert(PD % 2 == 0, "the table entries alternate between two sets by block parity within a ring pass");
    constexpr int kAr = 4;  // activation-fragment ring, MFMA steps
    static_assert(8 % kAr == 0, "the ring divides the eight MFMA steps of a block");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef __attribute__((address_space(3))) const gm_u32x2 lds_u32x2;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int hi = lane >> 5;
    const int64_t rows = a.n0 + a.n1;

    // ---- table: entry b, copy c at b * 256 + c * 8
    // (built in the first segment, once its first loads are in flight)
    auto build_table = [&]() {
        const uint32_t b = static_cast<uint32_t>(tid);
        gm_u32x2 e;
        if constexpr (Q2) {
            uint32_t q[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t c = (b >> (2 * f)) & 3u;
                q[f] = c == 0 ? 0xBF80u : (c == 2 ? 0x3F80u : 0u);  // bf16 -1, +1; codes 1 and 3 -> 0
            }
            e = gm_u32x2{q[0] | (q[1] << 16), q[2] | (q[3] << 16)};
        } else {
            uint32_t r = b, h[5];
#pragma unroll
            for (int n = 0; n < 5; ++n) {
                const uint32_t t = 3u * r;
                h[n] = trit_hi(t >> 8);
                r = t & 0xffu;
            }
            e = gm_u32x2{h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24),
                         h[4] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24)};
        }
#pragma unroll 8
        for (int i = 0; i < kRdTabCopies; ++i)
            *reinterpret_cast<gm_u32x2 *>(lds + b * 256 + ((b + i) & (kRdTabCopies - 1)) * 8) = e;
    };
    bool table_built = false;  // workgroup-uniform
    const uint32_t lc = static_cast<uint32_t>(lane & (kRdTabCopies - 1)) << 3;

    // ---- work split as in k_gemm_mfma: whole tiles first, then an equal
    // run of the remaining tiles' (tile, block) units, one segment per tile
    // touched.
    const int64_t G = gridDim.x, wg = blockIdx.x;
    const int64_t Gs = a.sk_wgs;  // workgroups [0, Gs) share the stream-K units
    const int64_t sk_lo = wg < Gs ? wg * a.sk_units / Gs : 0, sk_hi = wg < Gs ? (wg + 1) * a.sk_units / Gs : 0;
    int64_t jdp = 0, useg = sk_lo;
    while (jdp < a.dp_rounds || useg < sk_hi) {
        int64_t tile, kb0;
        int nblk, kslot = 0;
        bool full;
        if (jdp < a.dp_rounds) {  // whole tile wg + jdp G
            tile = wg + jdp * G;
            kb0 = 0;
            nblk = static_cast<int>(a.nb);
            full = true;
            ++jdp;
        } else {  // units [useg, uend) of stream-K tile t2
            const int64_t t2 = useg / a.nb;
            kb0 = useg - t2 * a.nb;
            const int64_t uend = (t2 + 1) * a.nb < sk_hi ? (t2 + 1) * a.nb : sk_hi;
            nblk = static_cast<int>(uend - useg);
            tile = a.dp_tiles + t2;
            full = kb0 == 0 && nblk == a.nb;
            kslot = useg == sk_lo ? 0 : 1;
            useg = uend;
        }
        const int last = nblk - 1;
        auto blk = [&](int i) -> int64_t { return kb0 + (i < last ? i : last); };
        const int64_t tn = tile / a.tiles_m, tm = tile - tn * a.tiles_m;
        const int64_t tile_n = tn * kGemmBN;
        const int64_t mt0 = tm * TM;
        const int64_t row0 = tm * a.prow;  // first row of the tile

        // ---- this lane's column
        const int64_t gcol = tile_n + wave * 32 + (lane & 31);
        const uint8_t *wcol = a.w0;
        int64_t sstride = 0;
        int64_t sc_off = 0;  // Q2: from the row's first record to its scale pair
        if (gcol < rows) {
            const bool first = gcol < a.n0;
            const int64_t rr = first ? gcol : gcol - a.n0;
            if constexpr (Q2) {
                // records of row i of a tile at 64 i, its scale pair at 2048 + 4 i
                const int64_t i = rr % kTileRows;
                wcol = (first ? a.w0 : a.w1) + (rr / kTileRows) * kPq2TileBytes + i * (kTileBlocks * kPq2CodeBytes);
                sstride = (first ? a.bands0 : a.bands1) * kPq2TileBytes;
                sc_off = kPq2TileCodeBytes + 4 * i - i * (kTileBlocks * kPq2CodeBytes);
            } else {
                wcol = (first ? a.w0 : a.w1) + (rr / kTileRows) * kTileBytes +
                       (rr % kTileRows) * (kTileBlocks * kBlockBytes);
                sstride = (first ? a.bands0 : a.bands1) * kTileBytes;
            }
        }

        struct WRegs {
            gm_u32x4 v;  // bytes 8 h .. 8 h + 15 (Q2: code bytes 16 h .. 16 h + 15)
            uint32_t w;  // bytes 24..27 (Q2: the row's two scales)
            int sh;      // Q2: 16 for the slice's second block
        };
        auto load_w = [&](WRegs &r, int64_t kb) {
            if constexpr (Q2) {
                const uint8_t *t = wcol + (kb >> 1) * sstride;
                const gm_u32x4a v = *reinterpret_cast<const gm_u32x4a *>(t + (kb & 1) * kPq2CodeBytes + 16 * hi);
                r.v = gm_u32x4{v[0], v[1], v[2], v[3]};
                r.w = *reinterpret_cast<const uint32_t *>(t + sc_off);
                r.sh = static_cast<int>(kb & 1) * 16;
            } else {
                const uint8_t *p = wcol + (kb >> 1) * sstride + (kb & 1) * kBlockBytes;
                const gm_u32x4a v = *reinterpret_cast<const gm_u32x4a *>(p + 8 * hi);
                r.v = gm_u32x4{v[0], v[1], v[2], v[3]};
                r.w = *reinterpret_cast<const uint32_t *>(p + 24);
                r.sh = 0;
            }
        };
        auto tab_read = [&](uint32_t w, int byte) -> gm_u32x2 {
            const uint32_t addr = __builtin_amdgcn_perm(lc, w, 0x0c0c0004u | (static_cast<uint32_t>(byte) << 8));
            return *reinterpret_cast<lds_u32x2 *>(static_cast<uintptr_t>(addr));
        };
        struct Ent {
            gm_u32x2 g[8];  // "first" bytes: 0-7 (lanes 0-31) or 16-23 (lanes 32-63)
            gm_u32x2 m[8];  // bytes 8-15
            gm_u32x2 t[2];  // bytes 24, 25
            float scale;    // the block's scale, halved (trits are stored as +-2)
        };
        auto tab_reads = [&](const WRegs &r, Ent &e) {
            if constexpr (Q2) {  // g: code bytes of steps 0-3, m: of steps 4-7
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e.g[i] = tab_read(r.v[0], i);
                    e.g[4 + i] = tab_read(r.v[1], i);
                    e.m[i] = tab_read(r.v[2], i);
                    e.m[4 + i] = tab_read(r.v[3], i);
                }
                e.scale = half_bits_to_float((r.w >> r.sh) & 0xffffu);
                return;
            }
            const uint32_t g0 = hi ? r.v[2] : r.v[0], g1 = hi ? r.v[3] : r.v[1];
            const uint32_t m0 = hi ? r.v[0] : r.v[2], m1 = hi ? r.v[1] : r.v[3];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e.g[i] = tab_read(g0, i);
                e.g[4 + i] = tab_read(g1, i);
                e.m[i] = tab_read(m0, i);
                e.m[4 + i] = tab_read(m1, i);
            }
            e.t[0] = tab_read(r.w, 0);
            e.t[1] = tab_read(r.w, 1);
            e.scale = 0.5f * half_bits_to_float(r.w >> 16);
        };
        // per-lane selectors of steps 5 and 6 (digit 0 / 3 and 1 / 4 of bytes 8-15)
        const uint32_t sel5 = hi ? rd_sel(3) : rd_sel(0);
        const uint32_t sel6 = hi ? rd_sel(0) : rd_sel(1);
        auto bfrag = [&](const Ent &e, int st) -> bf16x8 {
            gm_u32x4 o;
            if constexpr (Q2) {
                const gm_u32x2 *src = st < 4 ? e.g : e.m;
                const int j = 2 * (st & 3);
                o = gm_u32x4{src[j][0], src[j][1], src[j + 1][0], src[j + 1][1]};
                return __builtin_bit_cast(bf16x8, o);
            }
            if (st < 5) {
                const int c = st == 4 ? 1 : 0;
                const uint32_t sl = rd_sel(st == 4 ? 0 : st);
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(e.g[2 * q + 1][c], e.g[2 * q][c], sl);
            } else if (st < 7) {
                const int c = st == 6 ? 1 : 0;
                const uint32_t sl = st == 5 ? sel5 : sel6;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(e.m[2 * q + 1][c], e.m[2 * q][c], sl);
            } else {
                gm_u32x4 lo, f15;
#pragma unroll
                for (int q = 0; q < 4; ++q) lo[q] = __builtin_amdgcn_perm(e.m[2 * q + 1][0], e.m[2 * q][0], rd_sel(2));
                f15[0] = __builtin_amdgcn_perm(e.t[0][0], e.t[0][0], 0x010c000cu);
                f15[1] = __builtin_amdgcn_perm(e.t[0][0], e.t[0][0], 0x030c020cu);
                f15[2] = __builtin_amdgcn_perm(e.t[1][0], e.t[0][1], 0x040c000cu);
                f15[3] = __builtin_amdgcn_perm(e.t[1][0], e.t[1][0], 0x020c010cu);
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = hi ? f15[q] : lo[q];
            }
            return __builtin_bit_cast(bf16x8, o);
        };

        // A lane whose row is padding (row >= m) reads the fragment of row 0
        // of its tile instead: its MFMA output row is never stored, and the
        // read shares the live lanes' cache lines (no traffic for padding).
        const uint16_t *xw[TM];
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const bool live_row = (mt0 + m) * 32 + (lane & 31) < a.m;
            xw[m] = a.xf + (((mt0 + m) * a.nb * 8 * kWave) + (live_row ? lane : (lane & 32))) * 8;
        }
        auto load_a = [&](gm_u32x4 (&f)[TM], int64_t kb, int st) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
                f[m] = *reinterpret_cast<const gm_u32x4 *>(xw[m] + (kb * 8 + st) * kWave * 8);
        };
        // LDS-staged activations: thread tid < 128 LR owns piece tid = (step,
        // half, row) of each block (a padding row loads row 0's piece)
        constexpr bool LA = rd_lds_a(TM, LR);
        constexpr int kPieces = 8 * 2 * 8 * LR;
        char *abuf = lds + kRdLds;
        const bool a_loader = tid < kPieces;  // wave-uniform (kPieces is a multiple of 64)
        const uint16_t *apc = a.xf;
        {
            const int p = tid < kPieces ? tid : 0;
            const int st_p = p / (16 * LR), q = p % (16 * LR), hl = q / (8 * LR), row = q % (8 * LR);
            const int gl = hl * 32 + (mt0 * 32 + row < a.m ? row : 0);
            apc = a.xf + ((mt0 * a.nb * 8 + st_p) * kWave + gl) * 8;
        }
        const int arow = (lane & 31) < 8 * LR ? (lane & 31) : 0;
        auto load_piece = [&](int64_t kb) -> gm_u32x4 {
            return *reinterpret_cast<const gm_u32x4 *>(apc + kb * 8 * kWave * 8);
        };
        auto put_piece = [&](int slot, const gm_u32x4 &v) {
            *reinterpret_cast<gm_u32x4 *>(abuf + slot * rd_a_slot(LR) + tid * 16) = v;
        };
        auto read_a = [&](gm_u32x4 (&f)[TM], int slot, int st) {
            f[0] = *reinterpret_cast<const gm_u32x4 *>(abuf + slot * rd_a_slot(LR) +
                                                       ((st * 2 + hi) * 8 * LR + arow) * 16);
        };
        gm_u32x4 apiece = {};

        f32x16 acc[TM], part[TM];
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][r] = part[m][r] = 0.0f;
        float sc_prev = 0.0f;

        // ---- prologue: PD blocks of weights, the table entries of block 0 and
        //      kAr steps of activations in flight
        WRegs ring[PD];
#pragma unroll
        for (int p = 0; p < PD; ++p) load_w(ring[p], blk(p));
        gm_u32x4 afr[kAr][TM];
        if constexpr (LA) {
            // the previous segment's last reads are done before slot 0 is rewritten
            if (table_built) __syncthreads();
            gm_u32x4 a0 = {};
            if (a_loader) {
                a0 = load_piece(blk(0));
                apiece = load_piece(blk(1));
            }
            if (!table_built) {
                build_table();
                table_built = true;
            }
            if (a_loader) put_piece(0, a0);
            __syncthreads();
#pragma unroll
            for (int st = 0; st < kAr; ++st) read_a(afr[st], 0, st);
        } else {
#pragma unroll
            for (int st = 0; st < kAr; ++st) load_a(afr[st], blk(0), st);
            if (!table_built) {  // first segment: the table is built while its loads are in flight
                build_table();
                __syncthreads();
                table_built = true;
            }
        }
        Ent ent[2];
        tab_reads(ring[0], ent[0]);
        load_w(ring[0], blk(PD));

        // One block: eight MFMA steps on the fragments of ent[cur]; step 1 also
        // issues the table reads of the next block (into ent[cur ^ 1]) and
        // refills its weight slot; step 0 first folds the previous block's
        // partial into acc.
        auto iteration = [&](int i, Ent &cur, Ent &nxt, WRegs &rslot) {
            if constexpr (LA) {
                if (a_loader) {
                    put_piece((i + 1) & 1, apiece);  // block i + 1, loaded one block ago
                    apiece = load_piece(blk(i + 2));
                }
            }
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                // block i + 1's slot is complete (and block i - 1's reads of it
                // done) once every wave is past this point
                if constexpr (LA)
                    if (st == 8 - kAr) __syncthreads();
                const bf16x8 bv = bfrag(cur, st);
                gm_u32x4 (&ar)[TM] = afr[st % kAr];
#pragma unroll
                for (int m = 0; m < TM; ++m) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, ar[m]);
                    if (st == 0) {
#pragma unroll
                        for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r)
                            acc[m][r] = fmaf(part[m][r], sc_prev, acc[m][r]);
                        const f32x16 z = {};
                        part[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, z, 0, 0, 0);
                    } else {
                        part[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, part[m], 0, 0, 0);
                    }
                }
                if constexpr (LA) {
                    if (st + kAr < 8)
                        read_a(ar, i & 1, st + kAr);
                    else
                        read_a(ar, (i + 1) & 1, st + kAr - 8);
                } else {
                    if (st + kAr < 8)
                        load_a(ar, blk(i), st + kAr);
                    else
                        load_a(ar, blk(i + 1), st + kAr - 8);
                }
                if (st == 1) {
                    tab_reads(rslot, nxt);
                    load_w(rslot, blk(i + 1 + PD));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sc_prev = cur.scale;
        };

        for (int base = 0; base < nblk; base += PD) {
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                const int i = base + u;
                if (i >= nblk) break;
                iteration(i, ent[u & 1], ent[(u + 1) & 1], ring[(u + 1) % PD]);
            }
        }
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r) acc[m][r] = fmaf(part[m][r], sc_prev, acc[m][r]);

        // a segment over all blocks of its tile is final; any other is stored
        // as this workgroup's first (0) or last (1) partial for k_gemm_fix
        float *pp = a.part + (wg * 2 + kslot) * a.prow * kGemmBN;
        const int64_t col = gcol;
        // the row offsets below are the same in every segment; an opaque lane
        // index keeps the compiler from hoisting them (16 rows x 64-bit
        // offsets) out of the segment loop into live registers
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        if (col < rows) {
#pragma unroll
            for (int m = 0; m < TM; ++m) {
#pragma unroll
                for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r) {
                    const int64_t row = (mt0 + m) * 32 + 8 * (r / 4) + 4 * (lane_e / 32) + (r % 4);
                    if (row >= a.m) continue;
                    const float v = acc[m][r];
                    if (!full) {
                        pp[(row - row0) * kGemmBN + (col - tile_n)] = v;
                    } else if (col < a.n0) {
                        const int64_t o = row * a.n0 + col;
                        a.y0[o] = a.residual ? a.residual[o] + v : v;
                    } else {
                        a.y1[row * a.n1 + (col - a.n0)] = v;
                    }
                }
            }
        }
    }  // segments
}

// ---------------------------------------------------------------------------
// 8-bit activations on the int8 matrix cores (W2A8: "Why I Am Building
// Another Inference Engine", Level 5, integer kernels on int8 activations;
// Level 4, a BitNet layer's int8 activations ahead of its ternary matmuls).
// The register-decode kernel above with int8 operands: activations are the
// per-row quantised q (k_prep_frag W8 layout), trits are exact int8
// -1 / 0 / +1, v_mfma_i32_32x32x32_i8 sums each 128-weight block exactly in
// int32 (|sum| <= 128 * 127), and the block's sum is scaled by its fp16
// scale in fp32; every stored output row is multiplied by its step.
// Table (64 KB, 32 copies per half-row): row b holds, for byte value b,
// T_lo = [d0-1, d1-1, d2-1, d3-1] (int8) in bytes 0..127 and T_hi = d4-1
// in every byte in 128..255.  Lane l (column l % 32, half h = l / 32) loads
// bytes 12 h .. 12 h + 15 of its column's block and the dword at byte 24,
// and reads 27 entries per block; step s's B operand is then dwords
// t = 4 s .. 4 s + 3 of the gemm_i8_kperm order (t < 12: one T_lo each;
// t = 12: T_lo of byte 24, or T_hi of 24 and three digits of 25; t > 12:
// T_hi of four bytes, two v_perm each).
// ---------------------------------------------------------------------------
typedef int32_t gm_i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t gm_i32x16 __attribute__((ext_vector_type(16)));

template <int TM, int PD, int LR>
__global__ void __launch_bounds__(kRdThreads, 2) k_gemm_i8(GemmArgs a)
{
    static_assert(LR >= 1 && LR <= 4, "8-row groups of a 32-row tile");
    static_assert(PD % 2 == 0, "the table entries alternate between two sets by block parity within a ring pass");
    constexpr int kSteps = 4;  // MFMA steps of K = 32 per block
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int hi = lane >> 5;
    const int64_t rows = a.n0 + a.n1;
    const uint8_t *xq = reinterpret_cast<const uint8_t *>(a.xf);

    auto build_table = [&]() {  // thread b: entry b, every copy
        const uint32_t b = static_cast<uint32_t>(tid);
        const uint32_t v = (243u * b) >> 8;  // the byte's code; its base-3 digits, most significant first
        const uint32_t d[5] = {v / 81u, (v / 27u) % 3u, (v / 9u) % 3u, (v / 3u) % 3u, v % 3u};
        uint32_t lo = 0;
#pragma unroll
        for (int n = 0; n < 4; ++n) lo |= ((d[n] + 255u) & 0xffu) << (8 * n);  // d - 1 as an int8 byte
        const uint32_t h4 = ((d[4] + 255u) & 0xffu) * 0x01010101u;
        const gm_u32x4 elo = {lo, lo, lo, lo}, ehi = {h4, h4, h4, h4};
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
            *reinterpret_cast<gm_u32x4 *>(lds + b * 256 + c * 4) = elo;
            *reinterpret_cast<gm_u32x4 *>(lds + b * 256 + 128 + c * 4) = ehi;
        }
    };
    bool table_built = false;  // workgroup-uniform
    const uint32_t lc = static_cast<uint32_t>(lane & 31) << 2;

    const int64_t G = gridDim.x, wg = blockIdx.x;
    const int64_t Gs = a.sk_wgs;
    const int64_t sk_lo = wg < Gs ? wg * a.sk_units / Gs : 0, sk_hi = wg < Gs ? (wg + 1) * a.sk_units / Gs : 0;
    int64_t jdp = 0, useg = sk_lo;
    while (jdp < a.dp_rounds || useg < sk_hi) {
        int64_t tile, kb0;
        int nblk, kslot = 0;
        bool full;
        if (jdp < a.dp_rounds) {
            tile = wg + jdp * G;
            kb0 = 0;
            nblk = static_cast<int>(a.nb);
            full = true;
            ++jdp;
        } else {
            const int64_t t2 = useg / a.nb;
            kb0 = useg - t2 * a.nb;
            const int64_t uend = (t2 + 1) * a.nb < sk_hi ? (t2 + 1) * a.nb : sk_hi;
            nblk = static_cast<int>(uend - useg);
            tile = a.dp_tiles + t2;
            full = kb0 == 0 && nblk == a.nb;
            kslot = useg == sk_lo ? 0 : 1;
            useg = uend;
        }
        const int last = nblk - 1;
        auto blk = [&](int i) -> int64_t { return kb0 + (i < last ? i : last); };
        const int64_t tn = tile / a.tiles_m, tm = tile - tn * a.tiles_m;
        const int64_t tile_n = tn * kGemmBN;
        const int64_t mt0 = tm * TM;
        const int64_t row0 = tm * a.prow;

        const int64_t gcol = tile_n + wave * 32 + (lane & 31);
        const uint8_t *wcol = a.w0;
        int64_t sstride = 0;
        if (gcol < rows) {
            const bool first = gcol < a.n0;
            const int64_t rr = first ? gcol : gcol - a.n0;
            wcol = (first ? a.w0 : a.w1) + (rr / kTileRows) * kTileBytes + (rr % kTileRows) * (kTileBlocks * kBlockBytes);
            sstride = (first ? a.bands0 : a.bands1) * kTileBytes;
        }
        struct WRegs {
            gm_u32x4 v;  // bytes 12 h .. 12 h + 15
            uint32_t w;  // bytes 24..27
        };
        auto load_w = [&](WRegs &r, int64_t kb) {
            const uint8_t *p = wcol + (kb >> 1) * sstride + (kb & 1) * kBlockBytes;
            const gm_u32x4a v = *reinterpret_cast<const gm_u32x4a *>(p + 12 * hi);
            r.v = gm_u32x4{v[0], v[1], v[2], v[3]};
            r.w = *reinterpret_cast<const uint32_t *>(p + 24);
        };
        // LDS address of the entry of byte `byte` of dword w (T_lo; T_hi at + 128)
        auto addr = [&](uint32_t w, int byte) -> uint32_t {
            return __builtin_amdgcn_perm(lc, w, 0x0c0c0004u | (static_cast<uint32_t>(byte) << 8));
        };
        auto rd = [&](uint32_t ad, int off) -> uint32_t {
            return *reinterpret_cast<lds_u32 *>(static_cast<uintptr_t>(ad + off));
        };
        struct Ent {
            uint32_t lo[12], hi[12];  // bytes 12 h .. 12 h + 11
            uint32_t lo24, hi24, lo25;
            float scale;
        };
        auto tab_reads = [&](const WRegs &r, Ent &e) {
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                const uint32_t ad = addr(r.v[i >> 2], i & 3);
                e.lo[i] = rd(ad, 0);
                e.hi[i] = rd(ad, 128);
            }
            const uint32_t a24 = addr(r.w, 0), a25 = addr(r.w, 1);
            e.lo24 = rd(a24, 0);
            e.hi24 = rd(a24, 128);
            e.lo25 = rd(a25, 0);
            e.scale = half_bits_to_float(r.w >> 16);
        };
        auto bfrag = [&](const Ent &e, int st) -> gm_i32x4 {
            gm_i32x4 o;
            if (st < 3) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = static_cast<int32_t>(e.lo[4 * st + q]);
            } else {
                // t = 12: weights 120 + 4 h .. 123 + 4 h (byte 24 digits 0-3; or byte 24
                // digit 4 and byte 25 digits 0-2)
                o[0] = static_cast<int32_t>(hi ? __builtin_amdgcn_perm(e.lo25, e.hi24, 0x06050400u) : e.lo24);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const uint32_t p01 = __builtin_amdgcn_perm(e.hi[4 * i + 1], e.hi[4 * i], 0x0c0c0400u);
                    const uint32_t p23 = __builtin_amdgcn_perm(e.hi[4 * i + 3], e.hi[4 * i + 2], 0x04000c0cu);
                    o[1 + i] = static_cast<int32_t>(p01 | p23);
                }
            }
            return o;
        };
        // A lane whose row is padding (row >= m) reads row 0 of its tile
        // instead: its output row is never stored.
        const uint8_t *xw[TM];
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const bool live_row = (mt0 + m) * 32 + (lane & 31) < a.m;
            xw[m] = xq + ((mt0 + m) * a.nb * kSteps * kWave + (live_row ? lane : (lane & 32))) * 16;
        }
        auto load_a = [&](gm_i32x4 (&f)[TM], int64_t kb, int st) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
                f[m] = *reinterpret_cast<const gm_i32x4 *>(xw[m] + (kb * kSteps + st) * kWave * 16);
        };

        f32x16 acc[TM];
        gm_i32x16 part[TM];
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[m][r] = 0.0f;
                part[m][r] = 0;
            }
        float sc_prev = 0.0f;

        // prologue: PD blocks of weights, block 0's activations (all four
        // steps: the ring is one block deep) and block 0's table entries
        WRegs ring[PD];
#pragma unroll
        for (int p = 0; p < PD; ++p) load_w(ring[p], blk(p));
        gm_i32x4 afr[kSteps][TM];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) load_a(afr[st], blk(0), st);
        if (!table_built) {
            build_table();
            __syncthreads();
            table_built = true;
        }
        Ent ent[2];
        tab_reads(ring[0], ent[0]);
        load_w(ring[0], blk(PD));

        // One block: four MFMA steps; step 0 first folds the previous block's
        // int32 sum (times its scale) into acc, each step refills its
        // activation slot with the next block's, and step 1 issues the next
        // block's table reads and refills its weight slot.
        auto iteration = [&](int i, Ent &cur, Ent &nxt, WRegs &rslot) {
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                const gm_i32x4 bv = bfrag(cur, st);
                gm_i32x4 (&ar)[TM] = afr[st];
#pragma unroll
                for (int m = 0; m < TM; ++m) {
                    if (st == 0) {
#pragma unroll
                        for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r)
                            acc[m][r] = fmaf(static_cast<float>(part[m][r]), sc_prev, acc[m][r]);
                        const gm_i32x16 z = {};
                        part[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[m], bv, z, 0, 0, 0);
                    } else {
                        part[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[m], bv, part[m], 0, 0, 0);
                    }
                }
                load_a(ar, blk(i + 1), st);
                if (st == 1) {
                    tab_reads(rslot, nxt);
                    load_w(rslot, blk(i + 1 + PD));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sc_prev = cur.scale;
        };

        for (int base = 0; base < nblk; base += PD) {
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                const int i = base + u;
                if (i >= nblk) break;
                iteration(i, ent[u & 1], ent[(u + 1) & 1], ring[(u + 1) % PD]);
            }
        }
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r)
                acc[m][r] = fmaf(static_cast<float>(part[m][r]), sc_prev, acc[m][r]);

        // final tiles are stored, shared ones as partials for k_gemm_fix; both
        // already carry the row's step
        float *pp = a.part + (wg * 2 + kslot) * a.prow * kGemmBN;
        const int64_t col = gcol;
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        if (col < rows) {
#pragma unroll
            for (int m = 0; m < TM; ++m) {
#pragma unroll
                for (int r = 0; r < (m == TM - 1 ? 4 * LR : 16); ++r) {
                    const int64_t row = (mt0 + m) * 32 + 8 * (r / 4) + 4 * (lane_e / 32) + (r % 4);
                    if (row >= a.m) continue;
                    const float v = a.row_scale != nullptr ? acc[m][r] * a.row_scale[row] : acc[m][r];
                    if (!full) {
                        pp[(row - row0) * kGemmBN + (col - tile_n)] = v;
                    } else if (col < a.n0) {
                        const int64_t o = row * a.n0 + col;
                        a.y0[o] = a.residual ? a.residual[o] + v : v;
                    } else {
                        a.y1[row * a.n1 + (col - a.n0)] = v;
                    }
                }
            }
        }
    }  // segments
}

// Stream-K tiles that more than one workgroup touched: the sum of their
// partials in workgroup order (+ residual), routed to y0 / y1.  Grid:
// (tiles - dp_tiles) x ceil(prow / kFixRows); a thread adds 4 adjacent
// columns of one row.
constexpr int kFixRows = kEwThreads / (kGemmBN / 4);  // rows per workgroup: 8

__global__ void __launch_bounds__(kEwThreads) k_gemm_fix(GemmArgs a)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    // workgroup-uniform: which workgroups hold partials of this tile
    const int64_t G = a.sk_wgs, t = a.dp_tiles + blockIdx.x;
    const int64_t first_u = static_cast<int64_t>(blockIdx.x) * a.nb;
    const int64_t w_lo = gemm_owner(first_u, a.sk_units, G), w_hi = gemm_owner(first_u + a.nb - 1, a.sk_units, G);
    if (w_lo == w_hi) return;  // stored final by its one workgroup
    // w_lo's segment of this tile is its first unless its range began in an
    // earlier tile; every later workgroup's range begins inside this tile
    const int64_t k_lo = (w_lo * a.sk_units < first_u * G) ? 1 : 0;
    const int64_t tn = t / a.tiles_m, tm = t - tn * a.tiles_m;
    const int64_t rows = a.n0 + a.n1;
    const int64_t r = static_cast<int64_t>(blockIdx.y) * kFixRows + threadIdx.x / (kGemmBN / 4);
    const int64_t c = 4 * (threadIdx.x % (kGemmBN / 4));
    const int64_t row = tm * a.prow + r, col = tn * kGemmBN + c;
    if (r >= a.prow || row >= a.m || col >= rows) return;
    const float *p0 = a.part + r * kGemmBN + c;
    const int64_t seg = 2 * a.prow * kGemmBN;  // floats per workgroup (first and last partial)
    // the residual of the four columns is requested with the partials
    // (clamped indices; used only for columns of y0): requested after the
    // sum it would add dependent round trips to memory
    float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.residual != nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t cj = col + j < a.n0 ? col + j : a.n0 - 1;
            res[j] = a.residual[row * a.n0 + cj];
        }
    }
    f32x4 v = *reinterpret_cast<const f32x4 *>(p0 + w_lo * seg + k_lo * a.prow * kGemmBN);
    // the later workgroups' first partials, sixteen requests in flight at a
    // time (clamped indices, no branch around the loads), added in order: a
    // tile of the batch-8 down projection has up to 14 owners, one round trip
    constexpr int kFixBatch = 16;
    for (int64_t base = w_lo + 1; base <= w_hi; base += kFixBatch) {
        f32x4 q[kFixBatch];
#pragma unroll
        for (int j = 0; j < kFixBatch; ++j)
            q[j] = *reinterpret_cast<const f32x4 *>(p0 + (base + j <= w_hi ? base + j : w_hi) * seg);
#pragma unroll
        for (int j = 0; j < kFixBatch; ++j)
            if (base + j <= w_hi) v += q[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t cj = col + j;
        if (cj >= rows) break;
        if (cj < a.n0) {
            a.y0[row * a.n0 + cj] = a.residual ? res[j] + v[j] : v[j];
        } else {
            a.y1[row * a.n1 + (cj - a.n0)] = v[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kPlanCus = 256;   // compute units the grid is sized for
constexpr int kMinBlocks = 4;   // fewest units a workgroup takes
}  // namespace

GemmPlan gemm_plan(int64_t m, int64_t rows, int64_t k, bool rd_only)
{
    // cfg 0 / 1: register-decode kernel, 32 / 64 rows, two workgroups per
    // CU; cfg 2: LDS-decode kernel, 128 rows with 8 waves, one per CU.
    // Either way the grid fills the CUs once: each workgroup takes whole
    // tiles for the full rounds there are, then an equal run of the rest's
    // (tile, K block) units.
    static const int64_t kBm[3] = {32, 64, 128};
    static const int64_t kPerCu[3] = {2, 2, 1};
    GemmPlan p;
    p.cfg = m <= 32 ? 0 : (m <= 64 || rd_only ? 1 : 2);
    const int64_t bm = kBm[p.cfg];
    p.m_pad = (m + bm - 1) / bm * bm;
    p.nb = k / kBlockWeights;
    p.tiles_n = (rows + kGemmBN - 1) / kGemmBN;
    p.tiles_m = p.m_pad / bm;
    p.prow = p.tiles_m == 1 ? m : bm;
    if (m == 0 || rows == 0 || p.nb == 0) return p;
    const int64_t tiles = p.tiles_n * p.tiles_m;
    int64_t g = kPerCu[p.cfg] * kPlanCus;
    if (g > tiles * p.nb / kMinBlocks) g = tiles * p.nb / kMinBlocks;
    p.wgs = g < 1 ? 1 : g;
    // whole tiles for as many full rounds as there are, the rest shared
    p.dp_rounds = tiles / p.wgs;
    p.sk_tiles = tiles - p.dp_rounds * p.wgs;
    return p;
}

size_t gemm_frag_elems(const GemmPlan &p, int64_t k) { return static_cast<size_t>(p.m_pad) * static_cast<size_t>(k); }

size_t gemm_part_floats(const GemmPlan &p)
{
    return static_cast<size_t>(2 * p.wgs) * static_cast<size_t>(p.prow) * kGemmBN;
}

bool gemm_fold_ok(const GemmPlan &p)
{
    const int64_t units = p.sk_tiles * p.nb, G = units < p.wgs ? units : p.wgs;
    for (int64_t j = 0; j < p.sk_tiles; ++j) {
        const int64_t first_u = j * p.nb;
        const int64_t w_lo = ((first_u + 1) * G + units - 1) / units - 1;
        const int64_t w_hi = ((first_u + p.nb) * G + units - 1) / units - 1;
        if (w_hi - w_lo + 1 > kSkPre) return false;
    }
    return true;
}

SkView gemm_sk_view(const GemmPlan &p, const float *part)
{
    SkView v;
    v.part = part;
    v.prow = p.prow;
    v.tiles_m = p.tiles_m;
    v.nb = p.nb;
    v.dp_tiles = p.dp_rounds * p.wgs;
    v.sk_units = p.sk_tiles * p.nb;
    v.sk_wgs = v.sk_units < p.wgs ? v.sk_units : p.wgs;
    return v;
}

hipError_t launch_prep_frag(const float *x, const float *g, const float *u, int64_t m, int64_t k,
                            const float *signs, float rms_eps, const float *gain, uint16_t *xf, hipStream_t s,
                            const SkView &sk)
{
    const int64_t nchunks = m * ((k + kHadamard - 1) / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_prep_frag<false, false>), dim3(static_cast<unsigned>(nchunks)), dim3(kPrepThreads), 0, s, x,
                       g, u, k, signs, rms_eps, gain, xf, static_cast<float *>(nullptr), sk);
    return hipGetLastError();
}

hipError_t launch_prep_frag_pq2(const float *x, const float *g, const float *u, int64_t m, int64_t k,
                                const float *signs, float rms_eps, const float *gain, uint16_t *xf, hipStream_t s,
                                const SkView &sk)
{
    const int64_t nchunks = m * ((k + kHadamard - 1) / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_prep_frag<true, false>), dim3(static_cast<unsigned>(nchunks)), dim3(kPrepThreads), 0, s, x,
                       g, u, k, signs, rms_eps, gain, xf, static_cast<float *>(nullptr), sk);
    return hipGetLastError();
}

hipError_t launch_prep_frag_w8(const float *x, int64_t m, int64_t k, uint8_t *xq, float *step, hipStream_t s)
{
    const int64_t nchunks = m * ((k + kHadamard - 1) / kHadamard);
    if (nchunks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_prep_frag<false, true>), dim3(static_cast<unsigned>(nchunks)), dim3(kPrepThreads), 0, s, x,
                       static_cast<const float *>(nullptr), static_cast<const float *>(nullptr), k,
                       static_cast<const float *>(nullptr), 0.0f, static_cast<const float *>(nullptr),
                       reinterpret_cast<uint16_t *>(xq), step, SkView{});
    return hipGetLastError();
}

// Launches one GEMM kernel instance (dynamic LDS above the 64 KB default is
// enabled once per instance and device), with the profiling events attached
// to the dispatch when a caller armed them.
template <int WM, int WN, int TM, int TN, int PD>
static hipError_t gemm_dispatch(dim3 grid, hipStream_t s, const GemmArgs &args)
{
    static std::atomic<uint64_t> lds_done{0};
    const auto kernel = k_gemm_mfma<WM, WN, TM, TN, PD>;
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), kGemmLds, lds_done);
    if (e != hipSuccess) return e;
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL(kernel, grid, dim3(64 * WM * WN), static_cast<uint32_t>(kGemmLds), s, pe.start,
                              pe.stop, 0u, args);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL(kernel, grid, dim3(64 * WM * WN), kGemmLds, s, args);
    }
    return hipGetLastError();
}

template <int TM, int PD, int LR, bool Q2 = false>
static hipError_t gemm_rd_dispatch(dim3 grid, hipStream_t s, const GemmArgs &args)
{
    static std::atomic<uint64_t> lds_done{0};
    const auto kernel = k_gemm_rd<TM, PD, LR, Q2>;
    constexpr int lds = kRdLds + (rd_lds_a(TM, LR) ? 2 * rd_a_slot(LR) : 0);
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), lds, lds_done);
    if (e != hipSuccess) return e;
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL(kernel, grid, dim3(kRdThreads), static_cast<uint32_t>(lds), s, pe.start, pe.stop, 0u,
                              args);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL(kernel, grid, dim3(kRdThreads), lds, s, args);
    }
    return hipGetLastError();
}

static GemmArgs gemm_args(const GemmPlan &p, const uint16_t *xf, int64_t m, const uint8_t *w0, int64_t n0,
                          const uint8_t *w1, int64_t n1, float *y0, float *y1, const float *residual, float *part)
{
    GemmArgs a;
    a.row_scale = nullptr;
    a.xf = xf;
    a.w0 = w0;
    a.w1 = w1;
    a.n0 = n0;
    a.n1 = n1;
    a.bands0 = (n0 + kTileRows - 1) / kTileRows;
    a.bands1 = (n1 + kTileRows - 1) / kTileRows;
    a.y0 = y0;
    a.y1 = y1;
    a.residual = residual;
    a.part = part;
    a.m = m;
    a.nb = p.nb;
    a.tiles_m = p.tiles_m;
    a.prow = p.prow;
    a.wgs = p.wgs;
    a.dp_rounds = p.dp_rounds;
    a.dp_tiles = p.dp_rounds * p.wgs;
    a.sk_units = p.sk_tiles * p.nb;
    a.sk_wgs = a.sk_units < p.wgs ? a.sk_units : p.wgs;
    return a;
}

static hipError_t gemm_fix(const GemmPlan &p, const GemmArgs &a, hipStream_t s)
{
    if (p.sk_tiles == 0) return hipSuccess;
    const unsigned ey = static_cast<unsigned>((p.prow + kFixRows - 1) / kFixRows);
    hipLaunchKernelGGL(k_gemm_fix, dim3(static_cast<unsigned>(p.sk_tiles), ey), dim3(kEwThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan &p, const uint16_t *xf, int64_t m, const uint8_t *w0, int64_t n0,
                       const uint8_t *w1, int64_t n1, float *y0, float *y1, const float *residual, float *part,
                       hipStream_t s, bool fix)
{
    const int64_t rows = n0 + n1;
    if (rows == 0 || m == 0 || p.nb == 0) return hipSuccess;
    const GemmArgs a = gemm_args(p, xf, m, w0, n0, w1, n1, y0, y1, residual, part);
    const dim3 grid(static_cast<unsigned>(p.wgs));
    hipError_t e;
    if (p.cfg == 0) {
        // a weight ring of two blocks at m <= 16 (batch 8: the 5120 x 17408
        // GEMM 16.4 against 17.1 us), four above (m = 64: 44.7 against 49.9)
        if (m <= 8)
            e = gemm_rd_dispatch<1, 2, 1>(grid, s, a);
        else if (m <= 16)
            e = gemm_rd_dispatch<1, 2, 2>(grid, s, a);
        else
            e = gemm_rd_dispatch<1, 4, 4>(grid, s, a);
    } else if (p.cfg == 1) {
        e = gemm_rd_dispatch<2, 4, 4>(grid, s, a);
    } else {
        e = gemm_dispatch<4, 2, 1, 2, 3>(grid, s, a);
    }
    if (e != hipSuccess || !fix) return e;
    return gemm_fix(p, a, s);
}

hipError_t launch_gemm_pq2(const GemmPlan &p, const uint16_t *xf, int64_t m, const uint8_t *w0, int64_t n0,
                           const uint8_t *w1, int64_t n1, float *y0, float *y1, const float *residual, float *part,
                           hipStream_t s, bool fix)
{
    if (n0 + n1 == 0 || m == 0 || p.nb == 0) return hipSuccess;
    if (p.cfg > 1) return hipErrorInvalidValue;  // register-decode plans only (gemm_plan(..., true))
    const GemmArgs a = gemm_args(p, xf, m, w0, n0, w1, n1, y0, y1, residual, part);
    const dim3 grid(static_cast<unsigned>(p.wgs));
    hipError_t e;
    if (p.cfg == 0) {
        if (m <= 8)
            e = gemm_rd_dispatch<1, 4, 1, true>(grid, s, a);
        else if (m <= 16)
            e = gemm_rd_dispatch<1, 4, 2, true>(grid, s, a);
        else
            e = gemm_rd_dispatch<1, 4, 4, true>(grid, s, a);
    } else {
        e = gemm_rd_dispatch<2, 4, 4, true>(grid, s, a);
    }
    if (e != hipSuccess || !fix) return e;
    return gemm_fix(p, a, s);
}

template <int TM, int PD, int LR>
static hipError_t gemm_i8_dispatch(dim3 grid, hipStream_t s, const GemmArgs &args)
{
    static std::atomic<uint64_t> lds_done{0};
    const auto kernel = k_gemm_i8<TM, PD, LR>;
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), kRdLds, lds_done);
    if (e != hipSuccess) return e;
    ProfEvents &pe = prof_events();
    if (pe.start != nullptr) {
        hipExtLaunchKernelGGL(kernel, grid, dim3(kRdThreads), static_cast<uint32_t>(kRdLds), s, pe.start, pe.stop, 0u,
                              args);
        pe = ProfEvents{};
    } else {
        hipLaunchKernelGGL(kernel, grid, dim3(kRdThreads), kRdLds, s, args);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const GemmPlan &p, const uint8_t *xq, int64_t m, const uint8_t *w, int64_t n, float *y,
                          const float *row_scale, float *part, hipStream_t s)
{
    if (n == 0 || m == 0 || p.nb == 0) return hipSuccess;
    if (p.cfg > 1) return hipErrorInvalidValue;  // register-decode plans only (gemm_plan(..., true))
    GemmArgs a = gemm_args(p, reinterpret_cast<const uint16_t *>(xq), m, w, n, nullptr, 0, y, nullptr, nullptr, part);
    a.row_scale = row_scale;
    const dim3 grid(static_cast<unsigned>(p.wgs));
    hipError_t e;
    if (p.cfg == 0) {
        if (m <= 8)
            e = gemm_i8_dispatch<1, 4, 1>(grid, s, a);
        else if (m <= 16)
            e = gemm_i8_dispatch<1, 4, 2>(grid, s, a);
        else
            e = gemm_i8_dispatch<1, 4, 4>(grid, s, a);
    } else {
        e = gemm_i8_dispatch<2, 4, 4>(grid, s, a);
    }
    if (e != hipSuccess) return e;
    return gemm_fix(p, a, s);
}

}  // namespace ptq1
