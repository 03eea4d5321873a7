/*
 * fp8q_oracle.c -- plain, slow, CPU-only definition of the fine-grained FP8
 * linear-layer path.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library; the product path
 * (libfp8q.so and its binding) never does, and this file shares no code,
 * header, table or constant generator with it.
 *
 * Sources (the five reference web pages; cited by site and post id):
 *   page 1  why-be.why-be.co.kr, wr_id=65900
 *   page 2  xn--jj0bz6z98ct0a29q.com, wr_id=362465
 *   page 3  why-be.why-be.co.kr, wr_id=55081
 *   page 4  sunipension.com, wr_id=314414
 *   page 5  lolipop-pandahouse.ssl-lolipop.jp, wr_id=1899274
 *
 * What is computed and where it is stated:
 *   - activations are grouped and scaled per 1x128 tile (one token, 128
 *     channels), weights per 128x128 block (page 4, passage on Figure 7(a));
 *   - a small group shares one scale so that it adapts to the group's own
 *     maximum (page 1, passage on sharing exponent bits among grouped
 *     elements; page 3, passage on accommodating outliers);
 *   - the scale maps the group's maximum magnitude onto the largest FP8 value
 *     (page 1, passage on the common per-tensor practice, applied here per
 *     group);
 *   - cached FP8 activations are converted from 1x128 to 128x1 tiles for the
 *     backward pass (page 4, same passage as Figure 7(a); page 1, passage on
 *     caching Linear inputs in FP8);
 *   - the GEMM applies the dequantization scales to FP32 partial results at a
 *     fixed K interval (page 3, passage on promotion and Figure 7(b); page 2,
 *     passage on dequantization folded into the increased-precision
 *     accumulation).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - FP8 format: OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF NaN, max 448);
 *   - scale s = fl32(amax / 448), stored in fp32, used as the dequantization
 *     multiplier; q = enc(fl32(x / s)), both divisions correctly rounded fp32;
 *   - power-of-two variant (scale_mode 1): s = the smallest power of two with
 *     448 * s >= amax, at least 2^-127; then q = enc(fl32(x / s)) as above;
 *   - enc rounds to the nearest E4M3 magnitude, ties to the even code,
 *     saturates at 448, and copies the sign bit (so -0 and negative values that
 *     round to zero give 0x80);
 *   - s == 0 (all-zero tile or amax/448 underflowing) stores s = 0 and writes
 *     the signed zero of each input;
 *   - partial tiles take amax over their valid elements only;
 *   - the K interval of the GEMM is 128 (the largest interval that never
 *     crosses a scale boundary);
 *   - requantization consumes the cached codes and scales: v = fl32(dec(q)*s),
 *     then the quantizer above on 128x1 tiles of v.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off (no fast-math: every fp32 and fp64
 * operation must round exactly once, to nearest even, with subnormals kept).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads used by the OpenMP loops below (for reporting CPU timings). */
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n); }

/* ------------------------------------------------------------------------- */
/* E4M3FN codec                                                              */
/* ------------------------------------------------------------------------- */

/* Value of an E4M3FN code: sign bit 7, exponent bits 6..3 (bias 7), mantissa
 * bits 2..0.  Exponent field 0 is subnormal: m * 2^-9.  Code 0x7F/0xFF is NaN. */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* The 127 finite non-negative magnitudes, in code order (0x00..0x7E), which is
 * also increasing order of value. */
static double g_mag[127];
/* Value of every code, filled from oracle_e4m3_decode (a lookup in the GEMM
 * loops instead of a decode call per product; same values). */
static double g_dec[256];
static int g_mag_ready = 0;

static void build_mag_table(void)
{
    if (g_mag_ready)
        return;
    for (int c = 0; c < 256; ++c)
        g_dec[c] = oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 127; ++c)
        g_mag[c] = g_dec[c];
    g_mag_ready = 1;
}

/* Round a finite fp32 value to E4M3FN: nearest magnitude, ties to the code
 * whose mantissa LSB is 0, |y| >= 448 saturates to 448, sign bit copied. */
uint8_t oracle_e4m3_encode(float y)
{
    build_mag_table();
    uint32_t bits;
    memcpy(&bits, &y, 4);
    uint8_t sign = (uint8_t)((bits >> 31) << 7);
    double a = fabs((double)y);
    int code;
    if (a >= g_mag[126]) {
        code = 126;
    } else {
        /* largest lo with g_mag[lo] <= a  (binary search over increasing values) */
        int lo = 0, hi = 126;
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (g_mag[mid] <= a)
                lo = mid;
            else
                hi = mid;
        }
        /* a lies in [g_mag[lo], g_mag[hi]); the midpoint is exact in double */
        double mid = 0.5 * (g_mag[lo] + g_mag[hi]);
        if (a < mid)
            code = lo;
        else if (a > mid)
            code = hi;
        else
            code = (lo & 1) ? hi : lo; /* tie: even mantissa LSB */
    }
    return (uint8_t)(sign | (uint8_t)code);
}

void oracle_e4m3_encode_array(const float *y, int64_t n, uint8_t *out)
{
    build_mag_table();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(y[i]);
}

/* Encode every fp32 bit pattern in [first, first + count) (inclusive of sign
 * patterns); NaN and infinite patterns give 0xFF so that callers can skip them. */
void oracle_e4m3_encode_patterns(uint32_t first, int64_t count, uint8_t *out)
{
    build_mag_table();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t b = first + (uint32_t)i;
        float y;
        memcpy(&y, &b, 4);
        out[i] = isfinite(y) ? oracle_e4m3_encode(y) : (uint8_t)0xFF;
    }
}

/* ------------------------------------------------------------------------- */
/* Tile quantizer                                                            */
/* ------------------------------------------------------------------------- */

/*
 * Power-of-two scale of a tile (the variant whose scales are exactly
 * representable as an 8-bit exponent, E8M0, the scale format of block-scaled
 * matrix instructions): the smallest power of two s with 448 * s >= amax,
 * but not below 2^-127 (the smallest E8M0 value).  amax == 0 gives s = 0, as
 * in the fp32-scale rule.  The FP8 GEMM of the pages multiplies partial
 * results by the scales (page 3, passage on promotion and Figure 7(b)); with
 * power-of-two scales that multiplication is exact.
 * Written as its definition: start below the answer and step up.
 */
static float pow2_scale(float amax)
{
    if (amax == 0.0f)
        return 0.0f;
    int e = ilogb(amax) - 10; /* 448 * 2^e < 2^(e+9) <= amax / 2: too small */
    if (e < -127)
        e = -127;
    while (ldexp(448.0, e) < (double)amax)
        ++e;
    return (float)ldexp(1.0, e); /* exact: -127 <= e <= 120 */
}

/*
 * Quantize x[rows][cols] (row stride ldx, values already widened exactly to
 * fp32) in tiles of tr x tc elements.  Tile (I, J) covers rows [I*tr, ...)
 * and columns [J*tc, ...), clipped to the matrix.  For each tile:
 *     amax = max |x|,   s = fl32(amax / 448)  (scale_mode 0)
 *                       s = pow2_scale(amax)  (scale_mode 1),
 *     q = enc(fl32(x / s))
 * (codes are the signed zeros of x when s == 0).
 * Outputs: q[rows][cols] (stride ldq) in the input's orientation, and
 * s[I][J] with stride lds.
 */
void oracle_quantize_tiles_mode(const float *x, int64_t rows, int64_t cols, int64_t ldx,
                                int64_t tr, int64_t tc, int scale_mode, uint8_t *q, int64_t ldq,
                                float *s, int64_t lds)
{
    build_mag_table();
    int64_t nti = (rows + tr - 1) / tr, ntj = (cols + tc - 1) / tc;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t I = 0; I < nti; ++I) {
        for (int64_t J = 0; J < ntj; ++J) {
            int64_t r0 = I * tr, r1 = r0 + tr < rows ? r0 + tr : rows;
            int64_t c0 = J * tc, c1 = c0 + tc < cols ? c0 + tc : cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(x[r * ldx + c]);
                    if (a > amax)
                        amax = a;
                }
            float sc = scale_mode == 1 ? pow2_scale(amax) : amax / 448.0f;
            s[I * lds + J] = sc;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float v = x[r * ldx + c];
                    uint8_t code;
                    if (sc == 0.0f)
                        code = signbit(v) ? 0x80 : 0x00;
                    else
                        code = oracle_e4m3_encode(v / sc);
                    q[r * ldq + c] = code;
                }
        }
    }
}

void oracle_quantize_tiles(const float *x, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t tr, int64_t tc, uint8_t *q, int64_t ldq,
                           float *s, int64_t lds)
{
    oracle_quantize_tiles_mode(x, rows, cols, ldx, tr, tc, 0, q, ldq, s, lds);
}

/* v[r][c] = fl32(dec(q[r][c]) * s[r/tr][c/tc])  -- the dequantized value of a
 * stored code (exact decode, one fp32 rounding of the product). */
void oracle_dequantize_tiles(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                             int64_t tr, int64_t tc, const float *s, int64_t lds,
                             float *v, int64_t ldv)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float d = (float)oracle_e4m3_decode(q[r * ldq + c]); /* exact in fp32 */
            v[r * ldv + c] = d * s[(r / tr) * lds + (c / tc)];
        }
}

/*
 * 1x128 -> 128x1 conversion of cached FP8 activations (page 4, passage on
 * converting activations for the backward pass).  Input: codes q[rows][cols]
 * with 1x128 scales s1[rows][cols/128] (oracle orientation).  Output, in the
 * same orientation: codes q2[rows][cols] and 128x1 scales s2[rows/128][cols].
 */
void oracle_requant_1x128_to_128x1_mode(const uint8_t *q, int64_t rows, int64_t cols,
                                        const float *s1, int scale_mode, uint8_t *q2, float *s2)
{
    float *v = (float *)malloc(sizeof(float) * (size_t)rows * (size_t)cols);
    int64_t ntc = (cols + 127) / 128;
    oracle_dequantize_tiles(q, rows, cols, cols, 1, 128, s1, ntc, v, cols);
    oracle_quantize_tiles_mode(v, rows, cols, cols, 128, 1, scale_mode, q2, cols, s2, cols);
    free(v);
}

void oracle_requant_1x128_to_128x1(const uint8_t *q, int64_t rows, int64_t cols,
                                   const float *s1, uint8_t *q2, float *s2)
{
    oracle_requant_1x128_to_128x1_mode(q, rows, cols, s1, 0, q2, s2);
}

/* ------------------------------------------------------------------------- */
/* Block-scaled GEMM in FP64                                                 */
/* ------------------------------------------------------------------------- */

/*
 * One output element of C = A * B^T with per-128-K scales:
 *   C[m][n] = sum_kb  P_kb * (sa[m][kb] * sb(n, kb)),
 *   P_kb    = sum_{k in chunk kb} dec(qa[m][k]) * dec(qb[n][k])
 * P_kb is exact in fp64 (each product is a multiple of 2^-18 below 2^18 and
 * a 128-term sum stays below 2^53 units), sa*sb is exact in fp64, and the
 * chunk's contribution and the running sum each round once.
 * T[m][n] = sum_k |dec(qa)*sa * dec(qb)*sb| is returned as the error scale.
 * bscale_mode 0: sb(n, kb) = sb[(n/128)*ldsb + kb]   (128x128 weight blocks)
 * bscale_mode 1: sb(n, kb) = sb[n*ldsb + kb]         (one scale per row of B
 *                                                     per chunk: 128x1 tiles)
 * sa(m, kb) = sa[m*ldsa + kb].  K must be a multiple of 128.
 */
static void gemm_entry(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa,
                       const uint8_t *qb, int64_t ldb, const float *sb, int64_t ldsb,
                       int bscale_mode, int64_t K, int64_t m, int64_t n,
                       double *c_out, double *t_out)
{
    double acc = 0.0, tol = 0.0;
    for (int64_t kb = 0; kb < K / 128; ++kb) {
        double p = 0.0, pabs = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
            double prod = g_dec[qa[m * lda + k]] * g_dec[qb[n * ldb + k]];
            p += prod;
            pabs += fabs(prod);
        }
        double a_s = (double)sa[m * ldsa + kb];
        double b_s = bscale_mode == 0 ? (double)sb[(n / 128) * ldsb + kb] : (double)sb[n * ldsb + kb];
        double scl = a_s * b_s;
        acc += p * scl;
        tol += pabs * fabs(scl);
    }
    *c_out = acc;
    *t_out = tol;
}

/* Selected outputs: C and T at the pairs (idx_m[i], idx_n[i]). */
void oracle_gemm_entries(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa,
                         const uint8_t *qb, int64_t ldb, const float *sb, int64_t ldsb,
                         int bscale_mode, int64_t K, const int64_t *idx_m,
                         const int64_t *idx_n, int64_t count, double *c, double *t)
{
    build_mag_table();
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i)
        gemm_entry(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, bscale_mode, K, idx_m[i], idx_n[i],
                   &c[i], &t[i]);
}

/* Every output: C[M][N], T[M][N] (row-major, stride N). */
void oracle_gemm(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa,
                 const uint8_t *qb, int64_t ldb, const float *sb, int64_t ldsb,
                 int bscale_mode, int64_t M, int64_t N, int64_t K, double *c, double *t)
{
    build_mag_table();
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_entry(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, bscale_mode, K, m, n,
                       &c[m * N + n], &t[m * N + n]);
}

/*
 * Grouped GEMM for MoE experts: rows [off[e], off[e+1]) of A are multiplied by
 * expert e's weight B_e = qb + e*b_stride (128x128 block scales at
 * sb + e*sb_stride).  Selected outputs only; row m's expert is found by a
 * linear scan of the offsets.
 */
void oracle_grouped_gemm_entries(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa,
                                 const uint8_t *qb, int64_t ldb, int64_t b_stride,
                                 const float *sb, int64_t ldsb, int64_t sb_stride,
                                 const int32_t *off, int G, int64_t K,
                                 const int64_t *idx_m, const int64_t *idx_n, int64_t count,
                                 double *c, double *t)
{
    build_mag_table();
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = idx_m[i];
        int e = -1;
        for (int g = 0; g < G; ++g)
            if (m >= off[g] && m < off[g + 1]) {
                e = g;
                break;
            }
        if (e < 0) {
            c[i] = NAN;
            t[i] = NAN;
            continue;
        }
        gemm_entry(qa, lda, sa, ldsa, qb + e * b_stride, ldb, sb + e * sb_stride, ldsb, 0, K,
                   m, idx_n[i], &c[i], &t[i]);
    }
}

/* ------------------------------------------------------------------------- */
/* Dgrad in FP64                                                             */
/* ------------------------------------------------------------------------- */

/*
 * Activation gradient of the linear layer, dX = dY * W, with the same
 * fine-grained scaling: dY[m][n] carries 1x128 scales along n (sdy[m][n/128])
 * and W[n][k] its 128x128 block scales (sw[n/128][k/128]).  The contraction
 * runs over n in 128-wide chunks nb:
 *   dX[m][k] = sum_nb  (sdy[m][nb] * sw[nb][k/128]) * sum_{n in nb} dec(dy[m][n]) dec(w[n][k]).
 * The pages run the backward GEMMs in FP8 as the forward one (page 4,
 * passage on Figure 6); the Dgrad operand layout is this library's reading.
 * Written against W's own [N][K] layout (no transposed copy).  N must be a
 * multiple of 128.  T[m][k] = sum_n |each scaled product| as for the GEMM.
 */
static void dgrad_entry(const uint8_t *qdy, int64_t lddy, const float *sdy, int64_t ldsdy,
                        const uint8_t *qw, int64_t ldw, const float *sw, int64_t ldsw,
                        int64_t N, int64_t m, int64_t k, double *c_out, double *t_out)
{
    double acc = 0.0, tol = 0.0;
    for (int64_t nb = 0; nb < N / 128; ++nb) {
        double p = 0.0, pabs = 0.0;
        for (int64_t n = nb * 128; n < nb * 128 + 128; ++n) {
            double prod = g_dec[qdy[m * lddy + n]] * g_dec[qw[n * ldw + k]];
            p += prod;
            pabs += fabs(prod);
        }
        double scl = (double)sdy[m * ldsdy + nb] * (double)sw[nb * ldsw + k / 128];
        acc += p * scl;
        tol += pabs * fabs(scl);
    }
    *c_out = acc;
    *t_out = tol;
}

void oracle_dgrad_entries(const uint8_t *qdy, int64_t lddy, const float *sdy, int64_t ldsdy,
                          const uint8_t *qw, int64_t ldw, const float *sw, int64_t ldsw, int64_t N,
                          const int64_t *idx_m, const int64_t *idx_k, int64_t count, double *c, double *t)
{
    build_mag_table();
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i)
        dgrad_entry(qdy, lddy, sdy, ldsdy, qw, ldw, sw, ldsw, N, idx_m[i], idx_k[i], &c[i], &t[i]);
}

/* ------------------------------------------------------------------------- */
/* Unquantized product in FP64 (reporting only, not parity)                  */
/* ------------------------------------------------------------------------- */

/*
 * The product the quantized GEMM approximates, from the inputs before
 * quantization: C[m][n] = sum_k x[m][k] * w[n][k] and T[m][n] = sum_k
 * |x[m][k] * w[n][k]|, at the pairs (idx_m[i], idx_n[i]).  Inputs are fp32
 * values (bf16 inputs widen exactly); each product is exact in fp64 (24 x 24
 * significant bits) and each addition rounds once.  Used to report how far
 * the fine-grained and the per-tensor quantization land from the unquantized
 * result (page 1, passage on per-tensor scaling and its sensitivity to
 * outliers; page 3, passage on the fine-grained grouping that accommodates
 * them).
 */
void oracle_matmul_f32_entries(const float *x, int64_t ldx, const float *w, int64_t ldw, int64_t K,
                               const int64_t *idx_m, const int64_t *idx_n, int64_t count, double *c,
                               double *t)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        const float *xr = x + idx_m[i] * ldx, *wr = w + idx_n[i] * ldw;
        double acc = 0.0, tol = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = (double)xr[k] * (double)wr[k];
            acc += prod;
            tol += fabs(prod);
        }
        c[i] = acc;
        t[i] = tol;
    }
}
