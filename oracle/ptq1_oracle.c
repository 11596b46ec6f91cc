/*
 * ptq1_oracle.c -- plain, slow, fp64 CPU reference for the PTQ1_0 ternary
 * linear layer with the Walsh-Hadamard fold.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the bench's CPU
 * baseline leg load it.  It shares no source, header, table or helper with
 * the HIP path.
 *
 * Sources (page titles and sections; no code is printed on the pages):
 *   [B]  "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally",
 *        section "What Bonsai is": weights are -1, 0, +1 with one 16-bit
 *        scale per 128 weights; five trits are packed into a byte in base 3
 *        (1.75 bits per weight); every weight matrix is multiplied by a
 *        1024-wide Walsh-Hadamard butterfly with a sign pattern before
 *        quantising, so activations are rotated before every matmul of a
 *        folded weight and embedding rows are un-rotated after lookup.
 *   [F]  same page, section "What Ferrox does with it": trit n of a byte is
 *        floor(3^(n+1) u) - 3 floor(3^n u) with u = byte / 256 (digit n of u
 *        in base 3, n = 0 first).
 *   [S]  same page, section "Speed, and where it goes": the feed-forward
 *        block is gate, SwiGLU, down (gate and up share one input).
 *   [G]  "Why I Am Building Another Inference Engine", Level 4, Decision 4:
 *        a layer normalises, rotates, projects and adds the residual.
 *
 * Readings where the pages are silent:
 *   - weight 5i+n of a block lives in byte i, base-3 digit n (n = 0 most
 *     significant); digit value d maps to weight d - 1;
 *   - a block is 26 trit bytes (130 digit slots; slots 128 and 129 are
 *     padding, written as digit 1 and ignored on decode) followed by the
 *     fp16 (IEEE binary16) scale, little-endian: 28 bytes;
 *   - encoding picks the smallest byte whose code is v: b = ceil(256 v / 243);
 *   - the Hadamard matrix is Sylvester's, natural order, normalised by
 *     1/sqrt(1024); rotate applies the signs first: y = (1/32) H (s * x);
 *     unrotate is the transpose: x = s * ((1/32) H y);
 *   - one sign vector serves every 1024-wide chunk of a row;
 *   - SwiGLU is silu(gate) * up with silu(z) = z / (1 + exp(-z));
 *   - the stacked block takes an optional parameter-free RMS scale of its
 *     input, a = (mean(x^2) + eps)^(-1/2), before the rotation.
 *
 * Decoding here uses integer base-3 arithmetic, not the float formula of [F];
 * the tests check that the two agree on all 256 bytes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK_W 128     /* weights per block                       [B] */
#define ORC_TRIT_BYTES 26   /* ceil(128 / 5) bytes of five trits each  [B] */
#define ORC_BLOCK_BYTES 28  /* trit bytes + one 16-bit scale           [B] */
#define ORC_HAD 1024        /* Hadamard width                          [B] */

int orc_block_weights(void) { return ORC_BLOCK_W; }
int orc_block_trit_bytes(void) { return ORC_TRIT_BYTES; }
int orc_block_bytes(void) { return ORC_BLOCK_BYTES; }
int orc_hadamard_width(void) { return ORC_HAD; }

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* IEEE 754 binary16 bit pattern -> double (exact). */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);     /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* Byte -> five base-3 digits [B].  Integer route: the code carried by byte
 * b is v = floor(243 b / 256) (the base-3 value of u = b/256 truncated to
 * five digits), and digit n is floor(v / 3^(4-n)) mod 3. */
void orc_byte_digits(uint8_t b, int d[5])
{
    int v = (243 * (int)b) >> 8;
    int p = 81;
    for (int n = 0; n < 5; ++n) {
        d[n] = (v / p) % 3;
        p /= 3;
    }
}

/* Five digits -> byte: the smallest b with floor(243 b / 256) == v. */
uint8_t orc_digits_byte(const int d[5])
{
    int v = 0;
    for (int n = 0; n < 5; ++n) v = 3 * v + d[n];
    return (uint8_t)((256 * v + 242) / 243);
}

static int bad_shape(int64_t n, int64_t k)
{
    return n < 0 || k < 0 || (k % ORC_BLOCK_W) != 0;
}

/* trits int8 [n][k] in {-1,0,1}, scales fp16 bits [n][k/128] -> blocks
 * [n][k/128][28].  Returns 0, or -1 on a bad shape or a trit outside
 * {-1, 0, 1}. */
int orc_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k, uint8_t *blocks)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const int8_t *t = trits + r * k + b * ORC_BLOCK_W;
            uint8_t *out = blocks + (r * nb + b) * ORC_BLOCK_BYTES;
            for (int i = 0; i < ORC_TRIT_BYTES; ++i) {
                int d[5];
                for (int n5 = 0; n5 < 5; ++n5) {
                    int j = 5 * i + n5;
                    if (j < ORC_BLOCK_W) {
                        int tv = t[j];
                        if (tv < -1 || tv > 1) return -1;
                        d[n5] = tv + 1;
                    } else {
                        d[n5] = 1;  /* padding slot */
                    }
                }
                out[i] = orc_digits_byte(d);
            }
            uint16_t s = scales[r * nb + b];
            out[ORC_TRIT_BYTES] = (uint8_t)(s & 0xff);
            out[ORC_TRIT_BYTES + 1] = (uint8_t)(s >> 8);
        }
    }
    return 0;
}

/* Trit value (digit - 1) of weight j of a block. */
static int block_trit(const uint8_t *blk, int j)
{
    int d[5];
    orc_byte_digits(blk[j / 5], d);
    return d[j % 5] - 1;
}

static uint16_t block_scale_bits(const uint8_t *blk)
{
    return (uint16_t)(blk[ORC_TRIT_BYTES] | (blk[ORC_TRIT_BYTES + 1] << 8));
}

/* blocks -> trits int8 [n][k] and scales fp16 bits [n][k/128]. */
int orc_unpack(const uint8_t *blocks, int64_t n, int64_t k, int8_t *trits, uint16_t *scales)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (r * nb + b) * ORC_BLOCK_BYTES;
            for (int j = 0; j < ORC_BLOCK_W; ++j)
                trits[r * k + b * ORC_BLOCK_W + j] = (int8_t)block_trit(blk, j);
            scales[r * nb + b] = block_scale_bits(blk);
        }
    return 0;
}

/* w[r][k] = fp16(scale of its block) * trit, in fp64. */
int orc_dequant(const uint8_t *blocks, int64_t n, int64_t k, double *w)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (r * nb + b) * ORC_BLOCK_BYTES;
            double s = orc_f16_to_f64(block_scale_bits(blk));
            for (int j = 0; j < ORC_BLOCK_W; ++j)
                w[r * k + b * ORC_BLOCK_W + j] = s * (double)block_trit(blk, j);
        }
    return 0;
}

/* ---- PQ2_0: the 2-bit ternary format of "Why I Am Building Another
 * Inference Engine", Level 2 (two bits for every ternary weight and a
 * 16-bit scale for every 128 of them: 2.125 bits per weight).  Readings (the
 * page gives neither field order nor code map): weight 4i+n of a block is
 * the 2-bit field n (n = 0 least significant) of byte i; code q in {0,1,2}
 * is the weight q - 1; code 3 (never written) decodes as weight 0; the 32
 * code bytes are followed by the fp16 scale, little-endian: 34 bytes. */
#define ORC_PQ2_CODE_BYTES 32
#define ORC_PQ2_BLOCK_BYTES 34

int orc_pq2_block_bytes(void) { return ORC_PQ2_BLOCK_BYTES; }

/* Weight of 2-bit code q. */
static int pq2_weight(int q) { return q == 3 ? 0 : q - 1; }

/* trits int8 [n][k] in {-1,0,1}, scales fp16 bits [n][k/128] -> blocks
 * [n][k/128][34].  Returns 0, or -1 on a bad shape or a trit outside
 * {-1, 0, 1}. */
int orc_pq2_pack(const int8_t *trits, const uint16_t *scales, int64_t n, int64_t k, uint8_t *blocks)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const int8_t *t = trits + r * k + b * ORC_BLOCK_W;
            uint8_t *out = blocks + (r * nb + b) * ORC_PQ2_BLOCK_BYTES;
            for (int i = 0; i < ORC_PQ2_CODE_BYTES; ++i) {
                int byte = 0;
                for (int f = 0; f < 4; ++f) {
                    int tv = t[4 * i + f];
                    if (tv < -1 || tv > 1) return -1;
                    byte += (tv + 1) << (2 * f);
                }
                out[i] = (uint8_t)byte;
            }
            uint16_t s = scales[r * nb + b];
            out[ORC_PQ2_CODE_BYTES] = (uint8_t)(s & 0xff);
            out[ORC_PQ2_CODE_BYTES + 1] = (uint8_t)(s >> 8);
        }
    return 0;
}

static int pq2_block_trit(const uint8_t *blk, int j) { return pq2_weight((blk[j / 4] >> (2 * (j % 4))) & 3); }

static uint16_t pq2_scale_bits(const uint8_t *blk)
{
    return (uint16_t)(blk[ORC_PQ2_CODE_BYTES] | (blk[ORC_PQ2_CODE_BYTES + 1] << 8));
}

/* blocks -> trits int8 [n][k] and scales fp16 bits [n][k/128]. */
int orc_pq2_unpack(const uint8_t *blocks, int64_t n, int64_t k, int8_t *trits, uint16_t *scales)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (r * nb + b) * ORC_PQ2_BLOCK_BYTES;
            for (int j = 0; j < ORC_BLOCK_W; ++j)
                trits[r * k + b * ORC_BLOCK_W + j] = (int8_t)pq2_block_trit(blk, j);
            scales[r * nb + b] = pq2_scale_bits(blk);
        }
    return 0;
}

/* w[r][k] = fp16(scale of its block) * weight, in fp64. */
int orc_pq2_dequant(const uint8_t *blocks, int64_t n, int64_t k, double *w)
{
    if (bad_shape(n, k)) return -1;
    int64_t nb = k / ORC_BLOCK_W;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (r * nb + b) * ORC_PQ2_BLOCK_BYTES;
            double s = orc_f16_to_f64(pq2_scale_bits(blk));
            for (int j = 0; j < ORC_BLOCK_W; ++j)
                w[r * k + b * ORC_BLOCK_W + j] = s * (double)pq2_block_trit(blk, j);
        }
    return 0;
}

/* Sylvester Hadamard entry, natural order: (-1)^popcount(i & j). */
double orc_hadamard_entry(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
}

/* Dense rotation of each 1024-wide chunk of each row [B]:
 * y = (1/32) H (s * x).  k must be a multiple of 1024. */
int orc_rotate(const double *x, int64_t m, int64_t k, const double *signs, double *y)
{
    if (m < 0 || k < 0 || (k % ORC_HAD) != 0) return -1;
    int64_t nc = k / ORC_HAD;
#pragma omp parallel for schedule(static)
    for (int64_t rc = 0; rc < m * nc; ++rc) {
        const double *xc = x + rc * ORC_HAD;
        double *yc = y + rc * ORC_HAD;
        double *sx = (double *)malloc(sizeof(double) * ORC_HAD);
        for (int j = 0; j < ORC_HAD; ++j) sx[j] = signs[j] * xc[j];
        for (int i = 0; i < ORC_HAD; ++i) {
            double acc = 0.0;
            for (int j = 0; j < ORC_HAD; ++j) acc += orc_hadamard_entry(i, j) * sx[j];
            yc[i] = acc / 32.0;
        }
        free(sx);
    }
    return 0;
}

/* Inverse (= transpose) of orc_rotate: x = s * ((1/32) H y). */
int orc_unrotate(const double *y, int64_t m, int64_t k, const double *signs, double *x)
{
    if (m < 0 || k < 0 || (k % ORC_HAD) != 0) return -1;
    int64_t nc = k / ORC_HAD;
#pragma omp parallel for schedule(static)
    for (int64_t rc = 0; rc < m * nc; ++rc) {
        const double *yc = y + rc * ORC_HAD;
        double *xc = x + rc * ORC_HAD;
        for (int i = 0; i < ORC_HAD; ++i) {
            double acc = 0.0;
            for (int j = 0; j < ORC_HAD; ++j) acc += orc_hadamard_entry(i, j) * yc[j];
            xc[i] = signs[i] * (acc / 32.0);
        }
    }
    return 0;
}

/* Y[i][j] = sum_k xr[i][k] * W[rows[j]][k] for the dequantised W of the
 * packed matrix: the plain definition of a matvec (m = 1) or GEMM with
 * already rotated activations.  rows == NULL means all n rows (nrows = n). */
int orc_gemm_rows(const uint8_t *blocks, int64_t n, int64_t k, const double *xr, int64_t m,
                  const int64_t *rows, int64_t nrows, double *y)
{
    if (bad_shape(n, k) || m < 0) return -1;
    if (rows == NULL) nrows = n;
    int64_t nb = k / ORC_BLOCK_W;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        if (r < 0 || r >= n) { bad = 1; continue; }
        double *w = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (r * nb + b) * ORC_BLOCK_BYTES;
            double s = orc_f16_to_f64(block_scale_bits(blk));
            for (int q = 0; q < ORC_BLOCK_W; ++q)
                w[b * ORC_BLOCK_W + q] = s * (double)block_trit(blk, q);
        }
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int64_t q = 0; q < k; ++q) acc += xr[i * k + q] * w[q];
            y[i * nrows + j] = acc;
        }
        free(w);
    }
    return bad ? -1 : 0;
}

int orc_gemm(const uint8_t *blocks, int64_t n, int64_t k, const double *xr, int64_t m, double *y)
{
    return orc_gemm_rows(blocks, n, k, xr, m, NULL, n, y);
}

/* h = silu(g) * u, silu(z) = z / (1 + exp(-z))   [S] */
void orc_swiglu(const double *g, const double *u, int64_t len, double *h)
{
    for (int64_t i = 0; i < len; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* a = (mean(x^2) + eps)^(-1/2) per row of x [m][d]; eps <= 0 gives a = 1. */
void orc_rms_scale(const double *x, int64_t m, int64_t d, double eps, double *a)
{
    for (int64_t i = 0; i < m; ++i) {
        if (eps <= 0.0) { a[i] = 1.0; continue; }
        double ss = 0.0;
        for (int64_t q = 0; q < d; ++q) ss += x[i * d + q] * x[i * d + q];
        a[i] = 1.0 / sqrt(ss / (double)d + eps);
    }
}

/* One feed-forward block on x [m][d] (tokens in rows):
 *   a  = RMS scale of x (or 1); gain [d] the norm's per-channel weight (NULL: 1)
 *   xr = rotate(a * gain * x);  g = Wg xr;  u = Wu xr   (Wg, Wu: [f][d] packed)
 *   h  = silu(g) * u;    hr = rotate(h)
 *   x_out = x + Wd hr                            (Wd: [d][f] packed)
 * [B] rotate before every folded matmul; [S] gate, SwiGLU, down; [G] add,
 * and the layer's norm with its own weight ahead of the rotation (Level 4). */
int orc_ffn_block(const double *x, int64_t m, int64_t d, int64_t f,
                  const uint8_t *wg, const uint8_t *wu, const uint8_t *wd,
                  const double *signs, double rms_eps, const double *gain, double *x_out)
{
    if (m < 0 || d % ORC_HAD || f % ORC_HAD) return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    double *xa = (double *)malloc(sizeof(double) * (size_t)(m * d + 1));
    double *xr = (double *)malloc(sizeof(double) * (size_t)(m * d + 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(m * f + 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)(m * f + 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(m * f + 1));
    double *hr = (double *)malloc(sizeof(double) * (size_t)(m * f + 1));
    double *dn = (double *)malloc(sizeof(double) * (size_t)(m * d + 1));
    int rc = 0;
    orc_rms_scale(x, m, d, rms_eps, a);
    for (int64_t i = 0; i < m; ++i)
        for (int64_t q = 0; q < d; ++q) xa[i * d + q] = a[i] * (gain ? gain[q] : 1.0) * x[i * d + q];
    rc |= orc_rotate(xa, m, d, signs, xr);
    rc |= orc_gemm(wg, f, d, xr, m, g);
    rc |= orc_gemm(wu, f, d, xr, m, u);
    orc_swiglu(g, u, m * f, h);
    rc |= orc_rotate(h, m, f, signs, hr);
    rc |= orc_gemm(wd, d, f, hr, m, dn);
    for (int64_t i = 0; i < m * d; ++i) x_out[i] = x[i] + dn[i];
    free(a); free(xa); free(xr); free(g); free(u); free(h); free(hr); free(dn);
    return rc ? -1 : 0;
}
