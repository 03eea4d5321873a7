/*
 * fp8q.h -- C ABI of the fine-grained FP8 linear-layer library for AMD
 * Instinct MI355X (gfx950).
 *
 * Method (five reference web pages, cited by site and post id):
 *   - activations are quantized per 1x128 tile (one token, 128 channels) and
 *     weights per 128x128 block (128 input x 128 output channels): page 4
 *     (sunipension.com, wr_id=314414), passage on Figure 7(a);
 *   - the scale of a group maps the group's largest magnitude onto the largest
 *     FP8 value: page 1 (why-be.why-be.co.kr, wr_id=65900), passage on the
 *     per-tensor practice, applied per group as in the passage on sharing
 *     exponent bits among small groups;
 *   - the FP8 GEMM accumulates each K interval in the matrix unit and then
 *     multiplies the partial result by its scales into an FP32 total: page 3
 *     (why-be.why-be.co.kr, wr_id=55081), passage on promotion to FP32 and
 *     Figure 7(b); page 2 (xn--jj0bz6z98ct0a29q.com, wr_id=362465), passage
 *     on dequantization folded into the increased-precision accumulation;
 *   - cached FP8 activations are converted from 1x128 to 128x1 tiles for the
 *     Wgrad GEMM, which runs in FP8: page 4, passages on Figure 7(a) and
 *     Figure 6; page 1, passage on caching Linear inputs in FP8.
 *
 * Numeric definition shared by every quantizer (OCP E4M3FN codes, max 448):
 *   amax = max |x| over the tile's valid elements,
 *   s    = fl32(amax / 448)                      (stored fp32 scale),
 *   q    = e4m3(fl32(x / s))   round to nearest even, saturate at +-448,
 *                              sign kept (-0 -> 0x80); s == 0 gives the
 *                              signed zero of x.
 * Dequantized value: dec(q) * s.  Quantized bytes and scales are deterministic
 * and bit-reproducible.
 *
 * Conventions for every entry point:
 *   - all data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns (the
 *     one kernel that needs scratch memory, split-K, takes it from the
 *     caller as a workspace argument);
 *   - `stream` is a hipStream_t (NULL = the null stream); work is enqueued
 *     asynchronously on it and the call returns without synchronizing;
 *   - arguments are validated on the host before anything is enqueued; on
 *     error nothing is launched and a nonzero fp8q_status is returned;
 *   - FP8Q_EHIP reports a launch failure (hipGetLastError after the launch);
 *   - leading dimensions ("ld*") are in elements; all matrices are row-major;
 *   - base pointers of code and input arrays must be 16-byte aligned and
 *     leading dimensions of code/input arrays multiples of 16 bytes; scale
 *     arrays need 4-byte alignment only;
 *   - empty problems (a zero dimension) are valid and launch nothing;
 *   - calls hold no global mutable state and may be made from several host
 *     threads; calls on one stream execute in order;
 *   - a call enqueues kernel launches only (no memset, copy or host
 *     synchronization), so a sequence of calls can be captured into a HIP
 *     graph on its stream and replayed; the replays read the buffers' current
 *     contents.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8Q_OK = 0,
    FP8Q_EINVAL = 1,      /* null pointer, unknown enum value */
    FP8Q_ESHAPE = 2,      /* negative dimension, leading dimension too small,
                             K not a multiple of 128 in a GEMM, bad offsets */
    FP8Q_EALIGN = 3,      /* misaligned base pointer or leading dimension */
    FP8Q_EUNSUPPORTED = 4,/* valid request this build does not implement */
    FP8Q_EHIP = 5         /* HIP launch error */
} fp8q_status;

typedef enum { FP8Q_F32 = 0, FP8Q_BF16 = 1 } fp8q_dtype;

typedef enum {
    /* q[rows][cols] (ldq >= cols), s[ceil(cols/128)][rows] (lds >= rows):
       the scale of row r, column chunk j is s[j*lds + r]. */
    FP8Q_TILE_1x128 = 0,
    /* 128x1 tiles, output transposed: q[cols][rows] (ldq >= rows),
       s[ceil(rows/128)][cols] (lds >= cols): the scale of column c, row
       chunk i is s[i*lds + c]. */
    FP8Q_TILE_128x1 = 1
} fp8q_tile;

typedef enum {
    /* one scale per 128x128 block of B: s_b[ceil(N/128)][K/128] (ldsb >= K/128) */
    FP8Q_BSCALE_BLOCK128 = 0,
    /* one scale per row of B per 128-wide K chunk: s_b[K/128][N] (ldsb >= N) */
    FP8Q_BSCALE_ROW = 1
} fp8q_bscale;

/*
 * Activation quantizer: x[rows][cols] (dtype x_dtype, row stride ldx) into
 * E4M3 codes with one fp32 scale per tile (1x128 or 128x1, see fp8q_tile).
 * Partial tiles at the right/bottom edge take amax over their valid elements.
 * The 128x1 form is used for the activation gradient of the Wgrad GEMM (one
 * scale per output channel per 128 tokens).
 */
int fp8q_quantize_act(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                      int tile, uint8_t *q, int64_t ldq, float *s, int64_t lds, void *stream);

/*
 * Weight quantizer: w[N][K] (dtype w_dtype, row stride ldw) into codes
 * q[N][K] (row stride ldq) with one fp32 scale per 128x128 block:
 * s[ceil(N/128)][ceil(K/128)] (row stride lds >= ceil(K/128)).
 */
int fp8q_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                         uint8_t *q, int64_t ldq, float *s, int64_t lds, void *stream);

/*
 * 1x128 -> 128x1 conversion of cached FP8 activations.
 * Input: codes q[rows][cols] (rows = tokens, cols = channels, stride ldq) with
 * 1x128 scales s[ceil(cols/128)][rows] (stride lds >= rows).
 * Each element is dequantized to v = fl32(dec(q) * s), then v is quantized per
 * 128x1 tile (128 tokens of one channel) with the rule above.
 * Output (transposed): qt[cols][rows] (stride ldqt >= rows) and
 * st[ceil(rows/128)][cols] (stride ldst >= cols).
 */
int fp8q_requant_transpose(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                           const float *s, int64_t lds, uint8_t *qt, int64_t ldqt,
                           float *st, int64_t ldst, void *stream);

/*
 * Transpose of cached 128x128-quantized weights, for the Dgrad GEMM
 * dX[M][K] = dY[M][N] * W[N][K] (the pages run the backward GEMMs in FP8,
 * page 4, sunipension.com wr_id=314414, passage on Figure 6; Dgrad's operand
 * layout is this library's reading).  Input: codes q[N][K] (stride ldq) and
 * block scales s[ceil(N/128)][ceil(K/128)] (stride lds), as written by
 * fp8q_quantize_weight.  Output: qt[K][N] (stride ldqt >= N) with
 * qt[k][n] = q[n][k], and st[ceil(K/128)][ceil(N/128)] (stride ldst) with
 * st[j][i] = s[i][j]: exactly the 128x128 quantization of W^T.  Dgrad is then
 * fp8q_gemm(dY codes [M][N] with 1x128 scales, qt, st, FP8Q_BSCALE_BLOCK128,
 * M, K, N, ...), which needs N % 128 == 0.  Pure byte and word moves: the
 * output is bit-exact.  Any N, K.
 */
int fp8q_transpose_weight(const uint8_t *q, int64_t N, int64_t K, int64_t ldq, const float *s,
                          int64_t lds, uint8_t *qt, int64_t ldqt, float *st, int64_t ldst,
                          void *stream);

/*
 * Block-scaled FP8 GEMM:  C[M][N] (=|+=) sum over 128-wide K chunks kb of
 *     s_a(m, kb) * s_b(n, kb) * sum_{k in kb} dec(A[m][k]) * dec(B[n][k])
 * A: codes [M][K] (stride lda), s_a[K/128][M] (stride ldsa >= M), i.e. the
 *    FP8Q_TILE_1x128 layout of fp8q_quantize_act;
 * B: codes [N][K] (stride ldb), scales per `bscale` (fp8q_bscale).
 *    BLOCK128 matches fp8q_quantize_weight; ROW matches the transposed
 *    output of fp8q_requant_transpose / FP8Q_TILE_128x1.
 * Each chunk's partial product is formed by the matrix cores in FP32 and then
 * multiplied by its two scales into an FP32 running total (one promotion per
 * chunk).  K must be a multiple of 128; lda and ldb below 2^24 (larger row
 * strides give FP8Q_EUNSUPPORTED).  c_dtype FP8Q_BF16 (round to nearest
 * even at the end) or FP8Q_F32; accumulate != 0 (fp32 output only) adds the
 * result to the existing C.  M and N are arbitrary.
 */
int fp8q_gemm(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
              const uint8_t *b, int64_t ldb, const float *sb, int64_t ldsb, int bscale,
              int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
              int accumulate, void *stream);

/*
 * Grouped block-scaled GEMM for MoE experts.  Rows [off[g], off[g+1]) of A
 * (grouped by expert) are multiplied by expert g's weight:
 *   C[m][n] = sum_kb s_a(m, kb) * s_b^g(n/128, kb) * P_kb(m, n)
 * A: codes [M_total][K] (stride lda), s_a[K/128][M_total] (stride ldsa);
 * B: codes [G][N][K] (row stride ldb, expert stride b_group_stride elements),
 *    block scales [G][ceil(N/128)][K/128] (row stride ldsb, expert stride
 *    sb_group_stride);
 * group_offsets: DEVICE int32[G+1], nondecreasing, off[0] = 0,
 *    off[G] = M_total (not checked on the host: they stay on the device so
 *    that no synchronization is needed after routing).  The kernel uses
 *    off'[0] = clamp(off[0], 0, M_total), off'[g+1] = clamp(off[g+1], off'[g],
 *    M_total), so offsets out of range or decreasing never make it read past
 *    A or write past C; rows outside [off'[0], off'[G]) are not written.
 *    Empty groups are valid.
 * C[M_total][N] (stride ldc), c_dtype FP8Q_BF16 or FP8Q_F32.
 */
int fp8q_grouped_gemm(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
                      const uint8_t *b, int64_t ldb, int64_t b_group_stride,
                      const float *sb, int64_t ldsb, int64_t sb_group_stride,
                      const int32_t *group_offsets, int G, int64_t M_total, int64_t N,
                      int64_t K, void *c, int c_dtype, int64_t ldc, void *stream);

/*
 * Scale rule of the *_ex quantizers.
 * FP8Q_SCALE_FP32: s = fl32(amax / 448), the rule of the entry points above.
 * FP8Q_SCALE_POW2: s = the smallest power of two with 448 * s >= amax, never
 *   below 2^-127; s = 0 for an all-zero tile.  Every such scale is an 8-bit
 *   exponent (E8M0, the scale format of the block-scaled matrix instructions
 *   of gfx950) and multiplying by it is exact, so a GEMM can fold it into its
 *   operands (FP8Q_GEMM_POW2_SCALES below).  Codes: q = e4m3(fl32(x / s)) as
 *   above; since amax <= 448 s nothing saturates, and the tile uses between
 *   half and all of the E4M3 range.  The pages scale each group by its own
 *   maximum (page 1, why-be.why-be.co.kr wr_id=65900, passage on sharing
 *   exponent bits among small groups); rounding that scale up to a power of
 *   two is this library's variant.  Requantization in this mode is exact
 *   except where a value falls into the E4M3 subnormal range.
 */
typedef enum { FP8Q_SCALE_FP32 = 0, FP8Q_SCALE_POW2 = 1 } fp8q_scale_mode;

/* fp8q_quantize_act with a scale rule (fp8q_scale_mode). */
int fp8q_quantize_act_ex(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                         int tile, uint8_t *q, int64_t ldq, float *s, int64_t lds, int scale_mode,
                         void *stream);

/* fp8q_quantize_weight with a scale rule (fp8q_scale_mode). */
int fp8q_quantize_weight_ex(const void *w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                            uint8_t *q, int64_t ldq, float *s, int64_t lds, int scale_mode,
                            void *stream);

/* fp8q_requant_transpose with a scale rule for the 128x1 output scales. */
int fp8q_requant_transpose_ex(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                              const float *s, int64_t lds, uint8_t *qt, int64_t ldqt,
                              float *st, int64_t ldst, int scale_mode, void *stream);

/*
 * Gather + 1x128 quantization for MoE dispatch in FP8 (the pages dispatch
 * activations in FP8 before the expert GEMMs: page 2,
 * xn--jj0bz6z98ct0a29q.com wr_id=362465, and page 3, why-be.why-be.co.kr
 * wr_id=55081, passages on FP8 dispatch).  Output row i is row
 * row_index[i] of x[rows_in][cols] (stride ldx), quantized per 1x128 tile
 * with `scale_mode`: q[rows_out][cols] (stride ldq), s[ceil(cols/128)][rows_out]
 * (stride lds >= rows_out), the layout fp8q_grouped_gemm reads.  One pass:
 * each gathered row is read once and its codes written once.  row_index is a
 * DEVICE int32[rows_out] array (not read on the host); an index outside
 * [0, rows_in) marks an empty slot and gives a zero row (codes 0x00,
 * scale 0).  Rows may repeat (top-k routing).
 */
int fp8q_gather_quantize_act(const void *x, int x_dtype, int64_t rows_in, int64_t cols, int64_t ldx,
                             const int32_t *row_index, int64_t rows_out, uint8_t *q, int64_t ldq,
                             float *s, int64_t lds, int scale_mode, void *stream);

/*
 * Matrix-core datapath flags of fp8q_gemm_ex / fp8q_grouped_gemm_ex (bitwise
 * OR; 0 selects the default datapath of fp8q_gemm).  Unknown bits give
 * FP8Q_EINVAL.
 *
 * Default (0): every chunk partial P_kb is formed by f16 matrix instructions
 *   on exactly converted codes (every E4M3 value is an f16 value); products
 *   are exact and the partial sums round like FP32 additions, so
 *   |C - C_exact| <= 1e-5 * sum_k |a_k b_k| s_a s_b (+ half an ulp for bf16 C).
 *
 * FP8Q_GEMM_MMA_FP8: P_kb comes from the native FP8 matrix instruction (one
 *   v_mfma_f32_16x16x128_f8f6f4 per 16x16 subtile and chunk), twice the
 *   matrix rate of the default.  That instruction keeps limited precision
 *   while it adds products, the same effect the pages describe for FP8 tensor
 *   cores (page 3, why-be.why-be.co.kr wr_id=55081, passage on limited
 *   accumulation precision and Figure 7(b)): each run of 8 adjacent K
 *   products is summed with an alignment window of about 14 bit positions
 *   below the run's largest product, and bits below the window are truncated
 *   toward zero.  Per run the loss is below 8 * 2^-13 * max|product|, so
 *   |C - C_exact| <= 2^-10 * sum_k |a_k b_k| s_a s_b + the default bound.
 *   The promotion to FP32 every 128 K still bounds its growth with K.
 */
#define FP8Q_GEMM_MMA_FP8 1u

/*
 * FP8Q_GEMM_POW2_SCALES: the caller guarantees that every scale of A and B is
 * a power of two (the FP8Q_SCALE_POW2 quantizers produce them); only the
 * exponent field of each fp32 scale is used, so other scales give wrong
 * results.  The scales then move into the operands exactly and the matrix
 * core accumulates the whole K with no promotion step (the product of two
 * power-of-two scales needs no FP32 multiply):
 *   alone: each code is converted to bf16 already multiplied by its scale
 *     (exact for scales in [2^-124, 2^119]) and bf16 matrix instructions
 *     accumulate exact products like FP32 additions: the default bound holds;
 *   with FP8Q_GEMM_MMA_FP8: the block-scaled FP8 instruction
 *     v_mfma_scale_f32_16x16x128_f8f6f4 applies the E8M0 scales in hardware
 *     at the FP8 matrix rate; its in-instruction truncation is that of
 *     FP8Q_GEMM_MMA_FP8, the accumulator adds like FP32, so the FP8 bound
 *     (2^-10 T + the default bound) holds for any K.
 */
#define FP8Q_GEMM_POW2_SCALES 2u

/* fp8q_gemm with a datapath selection (flags above). */
int fp8q_gemm_ex(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
                 const uint8_t *b, int64_t ldb, const float *sb, int64_t ldsb, int bscale,
                 int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                 int accumulate, unsigned flags, void *stream);

/*
 * Split-K form of fp8q_gemm_ex for contractions whose output has too few
 * 256x256 tiles to occupy the GPU (a long K with small M and N, such as
 * 1024 x 1024 x 65536: 16 tiles on 256 compute units).  The K chunks are
 * dealt to S slices of consecutive chunks; each slice forms its FP32 partial
 * result with the same per-chunk promotion as fp8q_gemm (page 3,
 * why-be.why-be.co.kr wr_id=55081, passage on promotion to FP32 at a fixed K
 * interval, Figure 7(b)) and writes it to `workspace`; a second kernel adds
 * the S partials in slice order (FP32) and writes C in c_dtype (accumulate
 * as for fp8q_gemm).  The bound of the selected datapath holds (the extra
 * FP32 additions are far below 1e-5 of sum|ab|), and a repeated call gives
 * bitwise the same C.
 * fp8q_gemm_splitk_workspace(M, N, K) gives the bytes the split needs, or 0
 * when the shape fills the GPU without splitting (the call then runs as
 * fp8q_gemm_ex and ignores the workspace).  workspace: DEVICE memory of at
 * least that many bytes, 256-byte aligned, owned by the caller, not read
 * before it is written, free for reuse once the call's work on `stream` has
 * finished; NULL with a nonzero need gives FP8Q_EINVAL, fewer bytes
 * FP8Q_ESHAPE.  The plan depends on the device's compute-unit count.
 */
int64_t fp8q_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K);

int fp8q_gemm_splitk(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
                     const uint8_t *b, int64_t ldb, const float *sb, int64_t ldsb, int bscale,
                     int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                     int accumulate, unsigned flags, void *workspace, int64_t workspace_bytes,
                     void *stream);

/* fp8q_grouped_gemm with a datapath selection (flags above). */
int fp8q_grouped_gemm_ex(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
                         const uint8_t *b, int64_t ldb, int64_t b_group_stride,
                         const float *sb, int64_t ldsb, int64_t sb_group_stride,
                         const int32_t *group_offsets, int G, int64_t M_total, int64_t N,
                         int64_t K, void *c, int c_dtype, int64_t ldc, unsigned flags,
                         void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * split-K GEMM of fp8q_gemm_splitk with its partials in a scratch array that
 * the library itself holds in device memory, FP8Q_SPLITK_SCRATCH_BYTES per
 * device for the life of the process (set up on the first call on each
 * device).  Same arguments as fp8q_gemm_splitk without the workspace; the
 * same slice plan, kernels and bits.  A shape whose plan needs more than
 * FP8Q_SPLITK_SCRATCH_BYTES (fp8q_gemm_splitk_workspace) gives
 * FP8Q_EUNSUPPORTED; on MI355X (256 compute units) no shape does.  Shapes
 * that need no split run the plain kernel.  Calls neither allocate nor free.
 * Every call on one device shares that device's scratch: calls whose work
 * overlaps in time on one device (other streams, other host threads) race
 * and give wrong results; calls ordered on one stream are safe.  The scratch
 * keeps the last call's partials; nothing reads it before writing it.
 * FP8Q_EHIP if the scratch cannot be located on the current device.
 */
#define FP8Q_SPLITK_SCRATCH_BYTES (64u << 20)

int fp8q_gemm_splitk_noalloc(const uint8_t *a, int64_t lda, const float *sa, int64_t ldsa,
                             const uint8_t *b, int64_t ldb, const float *sb, int64_t ldsb, int bscale,
                             int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                             int accumulate, unsigned flags, void *stream);

/*
 * Measurement support (not part of the method): the shader clock under load.
 * One wave waits `ticks` ticks of the constant-rate real-time counter
 * (1 .. 1e8) and counts the shader-clock cycles that pass meanwhile; enqueued
 * on a second stream while other kernels run, out[1] / out[0] * out[2] kHz is
 * the clock of the compute unit it ran on.  out: DEVICE uint64[3] (8-byte
 * aligned): out[0] real-time ticks elapsed, out[1] shader-clock cycles,
 * out[2] real-time counter rate in kHz (0 if the runtime does not report it).
 */
int fp8q_clock_probe(uint64_t *out, int64_t ticks, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *fp8q_strerror(int status);

/* Library version: major*10000 + minor*100 + patch. */
int fp8q_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
