/*
 * oracle_driver.c -- runs every function of oracle/fp8q_oracle.c on ragged
 * shapes with buffers of exactly the documented sizes, built with the host
 * sanitizers (an out-of-bounds access, a use of uninitialised scale memory
 * through a wrong index, or undefined behaviour aborts the run), and checks
 * a few values that the definitions fix.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float y);
void oracle_e4m3_encode_array(const float *y, int64_t n, uint8_t *out);
void oracle_e4m3_encode_patterns(uint32_t first, int64_t count, uint8_t *out);
void oracle_quantize_tiles_mode(const float *x, int64_t rows, int64_t cols, int64_t ldx, int64_t tr, int64_t tc,
                                int scale_mode, uint8_t *q, int64_t ldq, float *s, int64_t lds);
void oracle_dequantize_tiles(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq, int64_t tr, int64_t tc,
                             const float *s, int64_t lds, float *v, int64_t ldv);
void oracle_requant_1x128_to_128x1_mode(const uint8_t *q, int64_t rows, int64_t cols, const float *s1,
                                        int scale_mode, uint8_t *q2, float *s2);
void oracle_gemm_entries(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa, const uint8_t *qb,
                         int64_t ldb, const float *sb, int64_t ldsb, int bscale_mode, int64_t K,
                         const int64_t *idx_m, const int64_t *idx_n, int64_t count, double *c, double *t);
void oracle_gemm(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa, const uint8_t *qb, int64_t ldb,
                 const float *sb, int64_t ldsb, int bscale_mode, int64_t M, int64_t N, int64_t K, double *c,
                 double *t);
void oracle_grouped_gemm_entries(const uint8_t *qa, int64_t lda, const float *sa, int64_t ldsa, const uint8_t *qb,
                                 int64_t ldb, int64_t b_stride, const float *sb, int64_t ldsb, int64_t sb_stride,
                                 const int32_t *off, int G, int64_t K, const int64_t *idx_m, const int64_t *idx_n,
                                 int64_t count, double *c, double *t);
void oracle_dgrad_entries(const uint8_t *qdy, int64_t lddy, const float *sdy, int64_t ldsdy, const uint8_t *qw,
                          int64_t ldw, const float *sw, int64_t ldsw, int64_t N, const int64_t *idx_m,
                          const int64_t *idx_k, int64_t count, double *c, double *t);
void oracle_matmul_f32_entries(const float *x, int64_t ldx, const float *w, int64_t ldw, int64_t K,
                               const int64_t *idx_m, const int64_t *idx_n, int64_t count, double *c, double *t);

static uint64_t st = 7;
static double urand(void) {
    st = st * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(st >> 11) * 0x1p-53;
}
static int fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);    \
            ++fails;                                               \
        }                                                          \
    } while (0)

static float *rand_f32(int64_t n) {
    float *p = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = (float)((urand() - 0.5) * ldexp(1.0, (int)(urand() * 20) - 10));
    return p;
}

int main(void) {
    CHECK(oracle_e4m3_encode(1.0f) == 0x38 && oracle_e4m3_encode(464.0f) == 0x7E);
    CHECK(oracle_e4m3_decode(0x7E) == 448.0 && isnan(oracle_e4m3_decode(0xFF)));
    uint8_t pat[4096];
    oracle_e4m3_encode_patterns(0x3F800000u - 2048u, 4096, pat);
    float ys[5] = {0.0f, -0.0f, 1e-30f, 500.0f, -3.0f};
    uint8_t yc[5];
    oracle_e4m3_encode_array(ys, 5, yc);
    CHECK(yc[1] == 0x80 && yc[3] == 0x7E);

    const int64_t shapes[][4] = {{3, 130, 1, 128}, {130, 3, 128, 1}, {257, 300, 128, 128}, {5, 40, 2, 40},
                                 {1, 1, 128, 128}, {129, 257, 1, 128}};
    for (int si = 0; si < 6; ++si) {
        const int64_t R = shapes[si][0], C = shapes[si][1], tr = shapes[si][2], tc = shapes[si][3];
        const int64_t ntr = (R + tr - 1) / tr, ntc = (C + tc - 1) / tc;
        for (int mode = 0; mode < 2; ++mode) {
            float *x = rand_f32(R * C);
            uint8_t *q = malloc((size_t)(R * C));
            float *s = malloc(sizeof(float) * (size_t)(ntr * ntc));
            float *v = malloc(sizeof(float) * (size_t)(R * C));
            oracle_quantize_tiles_mode(x, R, C, C, tr, tc, mode, q, C, s, ntc);
            oracle_dequantize_tiles(q, R, C, C, tr, tc, s, ntc, v, C);
            for (int64_t i = 0; i < R * C; ++i) {
                const float sc = s[(i / C / tr) * ntc + (i % C) / tc];
                CHECK(fabs((double)v[i] - x[i]) <= fmax(0x1p-4 * fabs((double)x[i]), 0x1p-10 * sc) + 1e-30);
            }
            free(x); free(q); free(s); free(v);
        }
    }
    /* requantization 1x128 -> 128x1 on a ragged matrix */
    {
        const int64_t R = 200, C = 300, ntc = 3, ntr = 2;
        float *x = rand_f32(R * C);
        uint8_t *q = malloc((size_t)(R * C)), *q2 = malloc((size_t)(R * C));
        float *s1 = malloc(sizeof(float) * (size_t)(R * ntc)), *s2 = malloc(sizeof(float) * (size_t)(ntr * C));
        oracle_quantize_tiles_mode(x, R, C, C, 1, 128, 0, q, C, s1, ntc);
        oracle_requant_1x128_to_128x1_mode(q, R, C, s1, 0, q2, s2);
        oracle_requant_1x128_to_128x1_mode(q, R, C, s1, 1, q2, s2);
        free(x); free(q); free(q2); free(s1); free(s2);
    }
    /* GEMMs: M = 5, N = 131 (a partial weight block), K = 384 */
    {
        const int64_t M = 5, N = 131, K = 384, nk = 3, nb = 2;
        float *a = rand_f32(M * K), *b = rand_f32(N * K);
        uint8_t *qa = malloc((size_t)(M * K)), *qb = malloc((size_t)(N * K));
        float *sa = malloc(sizeof(float) * (size_t)(M * nk)), *sb = malloc(sizeof(float) * (size_t)(nb * nk));
        float *sbr = malloc(sizeof(float) * (size_t)(N * nk));
        oracle_quantize_tiles_mode(a, M, K, K, 1, 128, 0, qa, K, sa, nk);
        oracle_quantize_tiles_mode(b, N, K, K, 128, 128, 0, qb, K, sb, nk);
        oracle_quantize_tiles_mode(b, N, K, K, 1, 128, 0, qb, K, sbr, nk);
        double *c = malloc(sizeof(double) * (size_t)(M * N)), *t = malloc(sizeof(double) * (size_t)(M * N));
        oracle_gemm(qa, K, sa, nk, qb, K, sb, nk, 0, M, N, K, c, t);
        oracle_gemm(qa, K, sa, nk, qb, K, sbr, nk, 1, M, N, K, c, t);
        int64_t im[4] = {0, 4, 2, 4}, in[4] = {0, 130, 128, 1};
        double ce[4], te[4];
        oracle_gemm_entries(qa, K, sa, nk, qb, K, sbr, nk, 1, 128, im, in, 4, ce, te);
        for (int i = 0; i < 4; ++i) CHECK(te[i] >= fabs(ce[i]));
        oracle_matmul_f32_entries(a, K, b, K, K, im, in, 4, ce, te);
        /* Dgrad: dY [5][256] 1x128, W [256][131] blocks */
        const int64_t Nd = 256, Kd = 131;
        float *dy = rand_f32(M * Nd), *w = rand_f32(Nd * Kd);
        uint8_t *qdy = malloc((size_t)(M * Nd)), *qw = malloc((size_t)(Nd * Kd));
        float *sdy = malloc(sizeof(float) * (size_t)(M * 2)), *sw = malloc(sizeof(float) * 2 * 2);
        oracle_quantize_tiles_mode(dy, M, Nd, Nd, 1, 128, 0, qdy, Nd, sdy, 2);
        oracle_quantize_tiles_mode(w, Nd, Kd, Kd, 128, 128, 0, qw, Kd, sw, 2);
        int64_t ik[4] = {0, 130, 128, 5};
        oracle_dgrad_entries(qdy, Nd, sdy, 2, qw, Kd, sw, 2, Nd, im, ik, 4, ce, te);
        /* grouped: 3 experts of 2, 0 and 3 rows; row 5 is outside every group */
        int32_t off[4] = {0, 2, 2, 5};
        uint8_t *qg = malloc((size_t)(3 * N * K));
        float *sg = malloc(sizeof(float) * (size_t)(3 * nb * nk));
        for (int g = 0; g < 3; ++g) oracle_quantize_tiles_mode(b, N, K, K, 128, 128, 0, qg + g * N * K, K,
                                                               sg + g * nb * nk, nk);
        int64_t gm[4] = {0, 1, 4, 3}, gn[4] = {0, 130, 7, 128};
        oracle_grouped_gemm_entries(qa, K, sa, nk, qg, K, N * K, sg, nk, nb * nk, off, 3, K, gm, gn, 4, ce, te);
        free(a); free(b); free(qa); free(qb); free(sa); free(sb); free(sbr); free(c); free(t);
        free(dy); free(w); free(qdy); free(qw); free(sdy); free(sw); free(qg); free(sg);
    }
    printf("oracle_driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
