// ptq1_launch.h -- internal launchers (host side), one per kernel family.
// Arguments are validated by the C ABI layer before any of these is called;
// each returns the hipError_t of its launch(es).
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <atomic>
#include <cstdint>

namespace ptq1 {

// Events for the next profiled launch (set by the C ABI's profiling hook,
// consumed and cleared by the launch it brackets): attached to that
// dispatch with hipExtLaunchKernel, so they time the kernel's execution and
// not the queue in front of it.
struct ProfEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents &prof_events();  // per host thread

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device, once
// per device (bit d of done_mask; calls that race set the same value).
hipError_t allow_dynamic_lds(const void *kernel, int bytes, std::atomic<uint64_t> &done_mask);

// The statically allocated per-device scratch buffer (scratch.hip): its
// device address on the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t{8} << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_device_ptr(void **ptr);

hipError_t launch_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k,
                       uint8_t *blocks, hipStream_t s);
hipError_t launch_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t s);
// packed [n][k] -> tiled layout (kTileRows x kTileBlocks tiles, zero padding)
hipError_t launch_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t s);

// PQ2_0: pack, dequant, and the reorder into its tiled layout (kPq2TileBytes
// per tile of 32 rows x 2 blocks)
hipError_t launch_pq2_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k, uint8_t *blocks,
                           hipStream_t s);
hipError_t launch_pq2_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t s);
hipError_t launch_pq2_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t s);

// rows of x [m][k] -> y, each 1024-chunk (1/32) H (signs * chunk)
hipError_t launch_rotate(const float *x, float *y, int64_t m, int64_t k, const float *signs,
                         hipStream_t s);
// out[i] = signs * (1/32) H table[ids ? ids[i] : i]  per chunk
hipError_t launch_unrotate_rows(const float *table, int64_t n_table, int64_t d, const int32_t *ids,
                                int64_t n_rows, const float *signs, float *out, hipStream_t s);

// ---- decode (m = 1) --------------------------------------------------------
hipError_t launch_swiglu(const float *g, const float *u, float *h, int64_t len, hipStream_t s);

// Lookup-table decode matvec over tiled weights, split over 256-wide
// K-slices: part[slice][matrix][row] (lut_part_floats floats) for one matrix
// (nmat = 1) or two sharing x (nmat = 2); x (times gain [k], if given)
// rotated per 1024-chunk when signs != nullptr, else used as given.
int64_t lut_nslices(int64_t k);
// W2A8 prefill: int8 MFMA operands of the per-row quantised x (k_prep_frag's
// W8 layout, m_pad * k bytes) and step[row]; then Y = step[row] * sum over
// blocks of scale * (int32 block sum), on a register-decode plan
// (gemm_plan(m, n, k, true)).
hipError_t launch_prep_frag_w8(const float *x, int64_t m, int64_t k, uint8_t *xq, float *step, hipStream_t s);
size_t lut_part_floats(int64_t n, int nmat, int64_t k);
// w8: 8-bit activations (W2A8) -- signs and gain are ignored; every
// workgroup takes max|x| itself, forms q = rint(x * float(127 / max|x|)),
// sums trits times q per block in int32 and stores step * sum_b scale_b * isum_b
// (step = max|x| / 127), so launch_lut_sum_rows gives the W2A8 product.
hipError_t launch_matvec_lut(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k,
                             const float *x, const float *signs, const float *gain, float *part, hipStream_t s,
                             bool w8 = false);
// The same partials with every trit peeled on the float pipeline (eight
// lanes per block), over the same tiled layout and slices.
hipError_t launch_matvec_peel(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k,
                              const float *x, const float *signs, const float *gain, float *part, hipStream_t s);
// The same lookup matvec over a PQ2_0 tiled matrix (one matrix): part as
// above, summed by launch_lut_sum_rows.
hipError_t launch_pq2_matvec(const uint8_t *w0, const uint8_t *w1, int nmat, int64_t n, int64_t k, const float *x,
                             const float *signs, const float *gain, float *part, hipStream_t s);
// y[r] = (residual ? residual[r] : 0) + sum over slices of part[s][r] (nmat = 1)
hipError_t launch_lut_sum_rows(const float *part, int64_t n, int64_t k, const float *residual, float *y,
                               hipStream_t s);
// nmat = 2 epilogue: g, u = a * sums (a = RMS scale of x_rms [d_rms], or 1
// when x_rms == nullptr), h = silu(g) u; any of g, u, h may be nullptr.
hipError_t launch_lut_gate_up_sum(const float *part, int64_t f, int64_t d_in, const float *x_rms, int64_t d_rms,
                                  float rms_eps, float *g, float *u, float *h, hipStream_t s);

// ---- prefill (m >= 1, bf16 MFMA) --------------------------------------------
// Shape of one GEMM launch: tile configuration (cfg 0/1 = 32/64 rows
// per workgroup, register decode; cfg 2 = 128 rows, LDS decode), padded
// activation rows, tiles, and the workgroups sharing the tiles x K blocks.
struct GemmPlan {
    int cfg = 0;
    int64_t m_pad = 0, tiles_n = 0, tiles_m = 0, nb = 0;
    int64_t prow = 0;  // rows of one row tile's partial (m when there is one row tile)
    int64_t wgs = 0;   // workgroups
    int64_t dp_rounds = 0, sk_tiles = 0;  // whole-tile rounds; tiles shared by (tile, block) units
};
// rd_only: register-decode configurations (32 or 64 rows per row tile) at any m
GemmPlan gemm_plan(int64_t m, int64_t rows, int64_t k, bool rd_only = false);
size_t gemm_frag_elems(const GemmPlan &p, int64_t k);  // bf16 A fragments
size_t gemm_part_floats(const GemmPlan &p);            // partial tiles of the work split
// The stream-K layout of one GEMM launch, for a consumer that adds the
// partials of shared tiles itself (the launch made with fix = false).
struct SkView {
    const float *part = nullptr;  // nullptr: no partials to add (y is final)
    int64_t prow = 0, tiles_m = 0, nb = 0, dp_tiles = 0, sk_units = 0, sk_wgs = 0;
};
// True when no shared tile of p spans more workgroups than the prep reads
// up front, so launch_prep_frag can take over p's fix-up.
bool gemm_fold_ok(const GemmPlan &p);
SkView gemm_sk_view(const GemmPlan &p, const float *part);
// xf = bf16 MFMA A fragments of R (a * gain * x) (rows < m only); a = RMS
// scale of x if rms_eps > 0, gain [k] or nullptr (1).  When g/u are given
// instead of x, the input is silu(g) * u (gain unused); with sk.part set, g
// and u are the outputs of a gate+up GEMM launched with fix = false (k = its
// n0 = n1): the prep adds the partials of its shared tiles (as the fix-up
// would, in the same order) and stores the finished g and u back.
hipError_t launch_prep_frag(const float *x, const float *g, const float *u, int64_t m, int64_t k,
                            const float *signs, float rms_eps, const float *gain, uint16_t *xf, hipStream_t s,
                            const SkView &sk = SkView{});
// y [m][rows] = A . W^T (+ residual [m][n0] if given), W tiled; the rows of
// the virtual matrix are w0's n0 rows, then w1's n1 rows (gate and up stacked),
// the first matrix's outputs in y0 [m][n0], the second's in y1 [m][n1].
// part: gemm_part_floats(p) floats of scratch.  fix = false leaves the
// shared tiles' partials in part for launch_prep_frag (no residual then).
hipError_t launch_gemm(const GemmPlan &p, const uint16_t *xf, int64_t m, const uint8_t *w0, int64_t n0,
                       const uint8_t *w1, int64_t n1, float *y0, float *y1, const float *residual, float *part,
                       hipStream_t s, bool fix = true);
// W2A8: y [m][n] = row_scale[row] * sum_b scale_b * (int32 block sum of
// trits x q), q the int8 activations of launch_prep_frag_w8 (their layout),
// W tiled; p from gemm_plan(m, n, k, true).
hipError_t launch_gemm_i8(const GemmPlan &p, const uint8_t *xq, int64_t m, const uint8_t *w, int64_t n, float *y,
                          const float *row_scale, float *part, hipStream_t s);
// PQ2_0: A fragments in the Q2 order (launch_prep_frag_pq2), y [m][n] =
// A . W^T over a PQ2_0 tiled matrix; p from gemm_plan(m, n, k, true).
hipError_t launch_prep_frag_pq2(const float *x, const float *g, const float *u, int64_t m, int64_t k,
                                const float *signs, float rms_eps, const float *gain, uint16_t *xf, hipStream_t s,
                                const SkView &sk = SkView{});
hipError_t launch_gemm_pq2(const GemmPlan &p, const uint16_t *xf, int64_t m, const uint8_t *w0, int64_t n0,
                           const uint8_t *w1, int64_t n1, float *y0, float *y1, const float *residual, float *part,
                           hipStream_t s, bool fix = true);

}  // namespace ptq1
