/*
 * ptq1.h -- C ABI of the MI355X (gfx950) PTQ1_0 ternary linear layer.
 *
 * The method: weights quantised to -1, 0, +1 with a 16-bit scale for every 128
 * weights, five trits packed into a byte in base 3 (1.75 bits per weight),
 * after every weight matrix was multiplied by a 1024-wide Walsh-Hadamard
 * butterfly with a sign pattern; at inference the same rotation is applied to
 * the activations before every folded matmul and undone on embedding rows
 * ("A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally", section
 * "What Bonsai is").  A trit is read from its byte on the float pipeline as
 * floor(3^(n+1) u) - 3 floor(3^n u), u = byte/256 (same page, section
 * "What Ferrox does with it").  Decode is a matvec, prefill a GEMM, and the
 * feed-forward block is gate and up, SwiGLU, down (section "Speed, and where
 * it goes").
 *
 * Layout of one PTQ1_0 block (28 bytes):
 *   bytes 0..25  trit bytes; weight 5i+n of the block is base-3 digit n of
 *                byte i (n = 0 most significant), digit d means weight d-1;
 *                byte 25 holds weights 125..127 in digits 0..2, digits 3..4
 *                are padding (written as 1, ignored when read);
 *   bytes 26..27 the block scale, IEEE binary16, little-endian.
 * A packed matrix [n][k] is row-major: row r is k/128 consecutive blocks.
 * Weight (r, c) = scale(r, c/128) * trit(r, c).
 *
 * Tiled layout (this library's device layout, not part of the format): the
 * same 28-byte blocks reordered so that each tile of 32 rows x 2 blocks
 * (256 weights of K) is 1792 contiguous bytes, K-slices outermost.  With
 * G = ceil(n/32) row bands, tile (g, t) -- rows 32g.., K-slice t -- starts at
 * byte (t*G + g) * 1792 and holds block j = 2t + b of row r = 32g + i at
 * byte (2i + b) * 28 of the tile; places past the matrix (r >= n or
 * j >= k/128) hold zero bytes.  The
 * matvec, gate/up, GEMM and feed-forward calls read weights in this layout
 * (ptq1_tile makes it from a packed matrix, once, at load time); pack
 * and dequant use the packed layout.
 *
 * Beyond PTQ1_0 with fp32 activations, two more numerics of the same layer:
 * the PQ2_0 format (pq2_*: two bits per weight, described before pq2_packed_bytes)
 * and 8-bit activations (ptq1_matvec_w2a8).
 *
 * Rotation R of a row x of width k (k a multiple of 1024): every 1024-wide
 * chunk c becomes (1/32) H (s * c), with H the natural-order Sylvester
 * Hadamard matrix and s the 1024 signs (one vector for every chunk).
 * R is orthogonal; the inverse applied to embedding rows is s * ((1/32) H c).
 *
 * Conventions for every call:
 *   - pointers are device pointers (hipMalloc'd or equivalent) unless stated;
 *     all memory is owned by the caller; weights are only read;
 *   - work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without waiting; a fault during execution surfaces at the caller's
 *     stream synchronisation, as usual in HIP;
 *   - on any status other than PTQ1_OK nothing has been enqueued (except
 *     PTQ1_ERR_HIP, which reports a failed launch);
 *   - ptq1_last_error() then names the refused argument (thread-local);
 *   - the library allocates no memory; calls that need scratch take a
 *     caller-owned workspace `ws` of at least the size the matching
 *     *_workspace_bytes() returns, 256-byte aligned, with any contents: it
 *     is scratch, written before it is read within each call, so one
 *     workspace may serve calls of any shape and entry point.  Calls that
 *     share a workspace must be ordered on one stream; two calls in flight
 *     at once must not share one.  The decode calls (matvec, gate_up,
 *     ffn_block with m = 1) take at most 2^20 output rows per matrix and
 *     tiled matrices below 2 GiB;
 *   - `float *` buffers must be 16-byte aligned, weights 16-byte aligned;
 *   - sizes are int64_t; products are checked for overflow.
 */
#ifndef PTQ1_H
#define PTQ1_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTQ1_BLOCK_WEIGHTS 128
#define PTQ1_TRIT_BYTES 26
#define PTQ1_BLOCK_BYTES 28
#define PTQ1_HADAMARD 1024
#define PTQ1_TILE_ROWS 32
#define PTQ1_TILE_BLOCKS 2

typedef enum ptq1_status {
    PTQ1_OK = 0,
    PTQ1_ERR_NULL = 1,        /* a required pointer is NULL                        */
    PTQ1_ERR_SHAPE = 2,       /* a size is negative or not a multiple it must be    */
    PTQ1_ERR_ALIGN = 3,       /* a pointer is not aligned as stated above          */
    PTQ1_ERR_OVERFLOW = 4,    /* a derived byte count or index overflows int64     */
    PTQ1_ERR_UNSUPPORTED = 5, /* a well-formed request this library does not run   */
    PTQ1_ERR_WORKSPACE = 6,   /* ws is NULL or smaller than *_workspace_bytes()    */
    PTQ1_ERR_ALIAS = 7,       /* an output overlaps an input it must not overlap   */
    PTQ1_ERR_HIP = 8          /* a HIP runtime call or kernel launch failed        */
} ptq1_status;

/* Human-readable name of a status.  Never NULL. */
const char *ptq1_status_string(ptq1_status s);

/* Message of the last non-OK status returned on this thread ("" if none).
 * Never NULL; valid until the next call on this thread. */
const char *ptq1_last_error(void);

/* Copies the compiled geometry {weights per block, trit bytes, block bytes,
 * Hadamard width, tile rows, tile blocks} into out[0..n) (n <= 6).
 * PTQ1_ERR_NULL / PTQ1_ERR_SHAPE. */
ptq1_status ptq1_geometry(int32_t *out, int32_t n);

/* Bytes of a packed [n][k] matrix: n * (k/128) * 28, or -1 if n < 0, k < 0,
 * k % 128 != 0 or the product overflows. */
int64_t ptq1_packed_bytes(int64_t n, int64_t k);

/* Codec encode ("What Bonsai is": five trits per byte in base 3, one 16-bit
 * scale per 128 weights).
 *   trits      int8 [n][k], values in {-1, 0, +1} (other values are clamped
 *              to the nearest of these);
 *   scales_f16 binary16 bit patterns [n][k/128], copied verbatim;
 *   blocks     output, ptq1_packed_bytes(n, k) bytes.
 * Each byte carries the code v = sum_n (t_n + 1) 3^(4-n) as the smallest
 * byte b with floor(243 b / 256) = v, i.e. b = ceil(256 v / 243).
 * Errors: NULL, SHAPE (k % 128), ALIGN (blocks), OVERFLOW. */
ptq1_status ptq1_pack(const int8_t *trits, const uint16_t *scales_f16, int64_t n, int64_t k,
                      uint8_t *blocks, hipStream_t stream);

/* Bytes of the tiled layout of an [n][k] matrix: ceil(n/32)*32 rows times
 * ceil(k/256)*2 blocks of 28 bytes (equal to ptq1_packed_bytes when n % 32
 * == 0 and k % 256 == 0), or -1 on a bad shape or overflow. */
int64_t ptq1_tiled_bytes(int64_t n, int64_t k);

/* Reorders a packed [n][k] matrix into the tiled layout described above
 * (bytes of every block copied unchanged, padding written as zeros).
 *   blocks  packed, ptq1_packed_bytes(n, k) bytes;
 *   tiled   output, ptq1_tiled_bytes(n, k) bytes, must not overlap blocks.
 * Errors: NULL, SHAPE (k % 128), ALIGN, ALIAS, OVERFLOW. */
ptq1_status ptq1_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t stream);

/* Codec decode ("What Ferrox does with it": digit n of u = b/256 read on the
 * float pipeline).  w [n][k] fp32 = binary16 scale * (digit - 1), exact.
 * Errors: NULL, SHAPE, ALIGN, OVERFLOW. */
ptq1_status ptq1_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t stream);

/* Rotation of activations ("What Bonsai is": the rotation applied to the
 * activations before every matmul of a folded weight).
 *   x, y  fp32 [m][k], k % 1024 == 0; y may equal x (in place), otherwise
 *         they must not overlap;
 *   signs1024  fp32 [1024], +-1.0 (other values are used as given and break
 *         orthogonality).
 * Errors: NULL, SHAPE (k % 1024), ALIGN, ALIAS (partial overlap), OVERFLOW. */
ptq1_status hadamard_rotate(const float *x, float *y, int64_t m, int64_t k, const float *signs1024,
                            hipStream_t stream);

/* Embedding lookup with the rotation undone ("What Bonsai is": undo the
 * rotation on the embedding table after each lookup).
 *   table  fp32 [n_table][d] row-major, rows stored rotated, d % 1024 == 0;
 *   ids    int32 [n_rows] device array of row indices, or NULL for rows
 *          0..n_rows-1; an id outside [0, n_table) yields a row of NaN;
 *   out    fp32 [n_rows][d]: out[i] = s * ((1/32) H table[ids[i]]) per chunk.
 * Errors: NULL, SHAPE (d % 1024, n_rows > n_table without ids), ALIGN,
 * ALIAS, OVERFLOW. */
ptq1_status hadamard_unrotate_rows(const float *table, int64_t n_table, int64_t d,
                                   const int32_t *ids, int64_t n_rows, const float *signs1024,
                                   float *out, hipStream_t stream);

/* Batch-1 decode matvec ("What Ferrox does with it": the decode matvec reads
 * every block once).
 *   y[r] = (residual ? residual[r] : 0) + sum_c W[r][c] * xr[c],
 *   xr = R x when signs1024 != NULL (k % 1024 == 0), else x as given.
 *   tiled   [n][k] in the tiled layout; x fp32 [k]; residual fp32 [n] or
 *   NULL; y fp32 [n] (y may equal residual, must not overlap x or tiled).
 * Trits are decoded through a per-slice table of byte-position x byte-value
 * partial dot products built from xr in 32-bit fixed point: each 256-wide
 * K-slice of xr is scaled by its own power of two so that max|xr| lies in
 * [2^22, 2^23) and rounded to integers once (an error of at most 2^-24 of the
 * slice's max|xr| per element); table entries and each block's sum are exact
 * int32, the block sum is scaled by its fp16 scale in fp32 and the rest is
 * fp32.  A NaN or an infinity in xr makes every output a NaN.  Two launches
 * (split-K partials per slice, then their sum in slice order).
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW, WORKSPACE. */
size_t ptq1_matvec_workspace_bytes(int64_t n, int64_t k);
ptq1_status ptq1_matvec(const uint8_t *tiled, int64_t n, int64_t k, const float *x,
                        const float *signs1024, const float *residual, float *y, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* The same matvec with every trit peeled on the float pipeline as the page
 * describes ("What Ferrox does with it": eight lanes share one 128-weight
 * block, each lane owns whole bytes, and a trit is floor(3^(n+1) u) -
 * 3 floor(3^n u), u = byte/256).  Same tiled matrix, results (to rounding
 * order and ptq1_matvec's fixed-point rounding of xr), workspace size and
 * errors as ptq1_matvec (its sums are fp32, so a NaN or an infinity
 * propagates as the float operations make it); kept as the page's own
 * decode, to be measured beside the table lookups. */
ptq1_status ptq1_matvec_float_peel(const uint8_t *tiled, int64_t n, int64_t k, const float *x,
                                   const float *signs1024, const float *residual, float *y, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* Gate and up projections of one token in one pass over a shared rotated
 * input ("Speed, and where it goes": paired projections fused into one GPU
 * submission).
 *   w_gate, w_up  tiled [f][d]; x fp32 [d]; g, u fp32 [f]:
 *   g = W_gate R x, u = W_up R x (R skipped when signs1024 == NULL), with
 * the table lookups and numerics of ptq1_matvec.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW, WORKSPACE. */
size_t ptq1_gate_up_workspace_bytes(int64_t f, int64_t d);
ptq1_status ptq1_gate_up(const uint8_t *w_gate, const uint8_t *w_up, int64_t f, int64_t d,
                         const float *x, const float *signs1024, float *g, float *u, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/* SwiGLU ("Speed, and where it goes": gate, SwiGLU, down):
 * h[i] = g[i] / (1 + exp(-g[i])) * u[i], fp32 [len].  h may equal g or u.
 * Errors: NULL, SHAPE (len < 0), ALIGN. */
ptq1_status ptq1_swiglu(const float *g, const float *u, float *h, int64_t len, hipStream_t stream);

/* Multi-token prefill GEMM ("What Ferrox does with it": a GEMM for prefill).
 *   Y [m][n] fp32 = bf16(R X) . W^T: X fp32 [m][k] is rotated (when
 *   signs1024 != NULL) and rounded to bf16 (nearest even); trits enter bf16
 *   MFMA exactly; each 128-weight block's partial sum is scaled by its fp16
 *   scale in fp32; accumulation is fp32.
 *   tiled [n][k] in the tiled layout; 1 <= m <= 65536; k % 128 == 0
 *   (k % 1024 == 0 with signs).
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW, WORKSPACE, UNSUPPORTED (m). */
size_t ptq1_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
ptq1_status ptq1_gemm(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m,
                      const float *signs1024, float *y, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/* One feed-forward block on m tokens ("Speed, and where it goes": the whole
 * block -- rotation, gate, SwiGLU, down -- enqueued as one sequence; "Why I
 * Am Building Another Inference Engine", Level 4: the layer's norm, with its
 * own weight, ahead of the rotation):
 *   a     = (mean(x^2) + rms_eps)^(-1/2) per token if rms_eps > 0, else 1
 *   xn    = a * rms_gain * x                      (rms_gain fp32 [d], NULL: 1)
 *   g, u  = W_gate R xn, W_up R xn                (W_gate, W_up tiled [f][d])
 *   h     = silu(g) * u
 *   x_out = x + W_down R h                        (W_down tiled [d][f])
 * m == 1 runs the table-lookup matvec path (numerics of ptq1_matvec), m >= 2
 * the bf16-MFMA GEMM path.
 * d % 1024 == 0, f % 1024 == 0; x_out may equal x; rms_gain, if given, is
 * 16-byte aligned and overlaps neither x_out nor ws.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW, WORKSPACE, UNSUPPORTED. */
size_t ptq1_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f);
ptq1_status ptq1_ffn_block(const float *x, float *x_out, int64_t m, int64_t d, int64_t f,
                           const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                           const float *signs1024, float rms_eps, const float *rms_gain, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* Where ptq1_ffn_block leaves the block's intermediate activations in its
 * workspace, so a caller can inspect each stage after the call ("A 27B model
 * in 5.5 GB: Bonsai ternary on Ferrox, locally", "Accuracy: measured, not
 * eyeballed": every execution path is compared stage by stage):
 *   offsets[0], offsets[1]  byte offsets of g and u, fp32 [m][f] (the gate
 *                           and up projections of the normalised input), for
 *                           m >= 2; -1 for m == 1;
 *   offsets[2]              byte offset of h = silu(g) * u, fp32 [f], for
 *                           m == 1; -1 for m >= 2 (there h is only formed in
 *                           bf16 inside the down projection's input).
 * They hold the values of the last call with this (m, d, f) until the
 * workspace is reused.  Errors: NULL, SHAPE (m < 1, d or f not a multiple of
 * 1024), UNSUPPORTED (m). */
ptq1_status ptq1_ffn_workspace_offsets(int64_t m, int64_t d, int64_t f, int64_t *offsets);

/* ptq1_ffn_block for callers that cannot allocate memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments, kernels, results and errors,
 * without ws / ws_bytes.  Its scratch is a buffer of 8 MiB (8388608 bytes)
 * that the library holds statically on every GPU it runs on, until the
 * process ends; a call whose ptq1_ffn_workspace_bytes(m, d, f) exceeds it is
 * refused with PTQ1_ERR_UNSUPPORTED before anything is enqueued (m = 1 up to
 * d = 8192, f = 28672; m <= 8 at d = 5120, f = 17408).  Nothing in it needs
 * to start at zero: every call writes the scratch it reads.  All calls on
 * one GPU share that buffer, so two calls that may overlap on one GPU (on
 * different streams, or from several host threads without ordering) race:
 * order them on one stream, or use ptq1_ffn_block with a workspace each.
 * The stage offsets of ptq1_ffn_workspace_offsets hold for this buffer too,
 * but it is not reachable from outside the library. */
ptq1_status ptq1_ffn_block_noalloc(const float *x, float *x_out, int64_t m, int64_t d, int64_t f,
                                   const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                                   const float *signs1024, float rms_eps, const float *rms_gain,
                                   hipStream_t stream);

/* ---- PQ2_0: the two-bit ternary format ("Why I Am Building Another
 * Inference Engine", Level 2: two bits per weight and a 16-bit scale for every
 * 128 weights, 2.125 bits per weight).  A block is 32 code bytes, weight
 * 4i + f in bits 2f..2f+1 of byte i (code q is the trit q - 1; code 3, never
 * written, reads as 0), then the binary16 scale, little-endian: 34 bytes.
 * The device layout for the matvec is tiled like PTQ1_0's (32 rows x 2
 * blocks per tile, tiles K-slice-major) with each tile holding its 64 code
 * records of 32 bytes first and then its 64 scales: 2176 bytes per tile. */

/* Bytes of a packed [n][k] PQ2_0 matrix: n * (k/128) * 34, or -1 if n < 0,
 * k < 0, k % 128 != 0 or the product overflows. */
int64_t pq2_packed_bytes(int64_t n, int64_t k);

/* Encode.  trits int8 [n][k] ({-1, 0, +1}; others clamped), scales_f16
 * binary16 bit patterns [n][k/128] (copied verbatim), blocks output of
 * pq2_packed_bytes(n, k) bytes, 16-byte aligned.
 * Errors: NULL, SHAPE (k % 128), ALIGN, ALIAS, OVERFLOW. */
ptq1_status pq2_pack(const int8_t *trits, const uint16_t *scales_f16, int64_t n, int64_t k, uint8_t *blocks,
                     hipStream_t stream);

/* Decode: w [n][k] fp32 = binary16 scale * trit, exact.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW. */
ptq1_status pq2_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t stream);

/* Bytes of the PQ2_0 tiled layout: ceil(n/32) * ceil(k/256) * 2176, or -1 on
 * a bad shape or overflow. */
int64_t pq2_tiled_bytes(int64_t n, int64_t k);

/* Packed -> tiled reorder (code bytes and scales copied unchanged, padding
 * written as zeros).  Both pointers 16-byte aligned, not overlapping.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW. */
ptq1_status pq2_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t stream);

/* Batch-1 decode matvec over a PQ2_0 tiled matrix, with the arguments,
 * results, workspace rule and errors of ptq1_matvec:
 *   y[r] = (residual ? residual[r] : 0) + sum_c W[r][c] * xr[c],
 *   xr = R x when signs1024 != NULL (k % 1024 == 0), else x as given.
 * Codes are decoded through a per-slice table of (code byte, byte value)
 * partial dot products over xr in the same 32-bit fixed point as
 * ptq1_matvec (exact int32 block sums; a NaN or infinity in xr makes every
 * output a NaN); split-K partials over 256-wide slices, then their sum in
 * slice order.  The tiled matrix must be below 2 GiB (UNSUPPORTED
 * otherwise). */
size_t pq2_matvec_workspace_bytes(int64_t n, int64_t k);
ptq1_status pq2_matvec(const uint8_t *tiled, int64_t n, int64_t k, const float *x, const float *signs1024,
                       const float *residual, float *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* Multi-token prefill GEMM over a PQ2_0 tiled matrix, with the arguments,
 * numerics, limits and errors of ptq1_gemm: Y [m][n] fp32 = bf16(R X) . W^T,
 * codes entering bf16 MFMA exactly as -1 / 0 / +1 and each block's partial
 * sum scaled by its fp16 scale in fp32. */
size_t pq2_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
ptq1_status pq2_gemm(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m, const float *signs1024,
                     float *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* The feed-forward block of ptq1_ffn_block over PQ2_0 tiled matrices: the
 * same arguments, numerics (m = 1: fixed-point table lookups as in
 * pq2_matvec; m >= 2: bf16 MFMA),
 * workspace rule and errors; every matrix must be below 2 GiB at m = 1. */
size_t pq2_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f);
ptq1_status pq2_ffn_block(const float *x, float *x_out, int64_t m, int64_t d, int64_t f, const uint8_t *w_gate,
                          const uint8_t *w_up, const uint8_t *w_down, const float *signs1024, float rms_eps,
                          const float *rms_gain, void *ws, size_t ws_bytes, hipStream_t stream);

/* The same stage offsets for pq2_ffn_block's workspace. */
ptq1_status pq2_ffn_workspace_offsets(int64_t m, int64_t d, int64_t f, int64_t *offsets);

/* Batch-1 decode matvec with 8-bit activations (W2A8: "Why I Am Building
 * Another Inference Engine", Level 5, the numerics of integer kernels; Level
 * 4, where a BitNet layer rounds its activations to int8 ahead of its ternary
 * matmuls):
 *   c = float(127 / max|x|) (0 when x is all zeros), q[i] = rint(x[i] * c) in
 *   fp32 (integers in [-127, 127], ties to even), step = max|x| / 127;
 *   y[r] = (residual ? residual[r] : 0) + step * sum_b s_rb * sum_{i in b} t_ri q_i.
 * x is used as given (rotate it first with hadamard_rotate for a folded
 * layer).  The per-block integer sums are exact; the block scales, the sum
 * over blocks and the step are fp32.  Same tiled matrix, residual and
 * aliasing rules as ptq1_matvec; k % 128 == 0, k > 0.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, OVERFLOW, WORKSPACE, UNSUPPORTED. */
size_t ptq1_matvec_w2a8_workspace_bytes(int64_t n, int64_t k);
ptq1_status ptq1_matvec_w2a8(const uint8_t *tiled, int64_t n, int64_t k, const float *x, const float *residual,
                             float *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* Prefill GEMM with 8-bit activations: each row of X [m][k] quantised as in
 * ptq1_matvec_w2a8 (its own absmax and step), the int8 rows multiplied with
 * the trits as int8 on the matrix cores (every 128-weight block summed
 * exactly in int32), each block sum scaled by its fp16 scale in fp32, and
 * row i of Y multiplied by its step:
 *   Y[i][r] = step_i * sum_b s_rb * sum_{c in b} t_rc q_ic.
 * X is used as given (no rotation).  Limits and errors as ptq1_gemm. */
size_t ptq1_gemm_w2a8_workspace_bytes(int64_t m, int64_t n, int64_t k);
ptq1_status ptq1_gemm_w2a8(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m, float *y, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* Profiling: attaches start[i] / stop[i] to the dispatch of the i-th of the
 * next `count` launches of one kernel family (hipExtLaunchKernel: they take
 * the kernel's own start and end times on its stream), so a caller can time
 * a kernel inside a composite call (ptq1_ffn_block) with events.  Families: "lut_matvec_2" (the
 * table-lookup matvec over two matrices: gate and up), "lut_matvec_1" (over
 * one matrix: ptq1_matvec, ptq1_matvec_w2a8, the down projection), "gemm" (the MFMA GEMM),
 * "pq2_matvec" (the PQ2_0 table-lookup matvec of pq2_matvec), "peel_matvec"
 * (the float-peel matvec of ptq1_matvec_float_peel); pq2_gemm's kernel
 * counts as "gemm".
 * Events are created and owned by the caller; both arrays must stay valid
 * until `count` launches have happened or the family is re-armed.  count =
 * 0 disarms.  Process-wide; not meant for concurrent use by several
 * threads.  Errors: NULL, SHAPE (count < 0), UNSUPPORTED (unknown name). */
ptq1_status ptq1_profile_arm(const char *kernel, hipEvent_t *start, hipEvent_t *stop, int32_t count);

/* Launches of `kernel` bracketed since it was last armed; -1 for an unknown
 * name. */
int32_t ptq1_profile_count(const char *kernel);

#ifdef __cplusplus
}
#endif

#endif /* PTQ1_H */
