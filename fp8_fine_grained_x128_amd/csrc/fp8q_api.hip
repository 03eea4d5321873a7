// fp8q_api.hip -- C ABI (include/fp8q.h): host-side validation, then one
// kernel launch on the caller's stream.  No allocation, no synchronization,
// no global mutable state.
#include <stdint.h>

#include <mutex>

#include "../../include/fp8q.h"
#include "launch.hpp"

// Device scratch of fp8q_gemm_splitk_noalloc: the split-K partials live here
// instead of in a caller workspace.  Each device that runs the library holds
// its own copy until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[FP8Q_SPLITK_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device (with that
// device current) on the first call; nullptr if the lookup fails.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();  // do not leave the error for the next call to report
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

constexpr int64_t kMaxGridY = 65535;
constexpr int kMaxGroups = 1024;
// The GEMM reads a tile's operand rows through a buffer descriptor with 32-bit
// offsets and a 32-bit record count: 256 rows * ld must stay below 2^32.
constexpr int64_t kMaxOperandLd = (int64_t(1) << 24) - 1;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int status_of(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_EHIP; }

inline int elem_bytes(int dtype) { return dtype == FP8Q_BF16 ? 2 : 4; }

inline bool valid_dtype(int d) { return d == FP8Q_F32 || d == FP8Q_BF16; }

inline bool valid_scale_mode(int m) { return m == FP8Q_SCALE_FP32 || m == FP8Q_SCALE_POW2; }

constexpr unsigned kKnownGemmFlags = FP8Q_GEMM_MMA_FP8 | FP8Q_GEMM_POW2_SCALES;

inline int datapath_of(unsigned flags) {
    const bool fp8 = (flags & FP8Q_GEMM_MMA_FP8) != 0u;
    if (flags & FP8Q_GEMM_POW2_SCALES) return fp8 ? fp8q::kMmaFp8Scaled : fp8q::kMmaBf16Fold;
    return fp8 ? fp8q::kMmaFp8 : fp8q::kMmaF16;
}

}  // namespace

extern "C" {

const char* fp8q_strerror(int status) {
    switch (status) {
        case FP8Q_OK: return "ok";
        case FP8Q_EINVAL: return "invalid argument (null pointer or unknown enum value)";
        case FP8Q_ESHAPE: return "invalid shape or leading dimension";
        case FP8Q_EALIGN: return "misaligned pointer or leading dimension";
        case FP8Q_EUNSUPPORTED: return "unsupported request";
        case FP8Q_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int fp8q_version(void) { return 200; }

static int quantize_act_impl(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int tile,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, int scale_mode, void* stream) {
    if (!valid_dtype(x_dtype) || (tile != FP8Q_TILE_1x128 && tile != FP8Q_TILE_128x1)) return FP8Q_EINVAL;
    if (!valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (rows < 0 || cols < 0) return FP8Q_ESHAPE;
    if (ldx < cols) return FP8Q_ESHAPE;
    if (tile == FP8Q_TILE_1x128) {
        if (ldq < cols || lds < rows) return FP8Q_ESHAPE;
    } else {
        if (ldq < rows || lds < cols) return FP8Q_ESHAPE;
    }
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_EINVAL;
    const int eb = elem_bytes(x_dtype);
    if (!aligned(x, 16) || (ldx * eb) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0 || !aligned(s, 4))
        return FP8Q_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int pow2 = scale_mode == FP8Q_SCALE_POW2;
    if (tile == FP8Q_TILE_1x128) {
        if (cdiv(cols, 512) > kMaxGridY) return FP8Q_EUNSUPPORTED;
        return status_of(fp8q::launch_quantize_1x128(x, x_dtype, rows, cols, ldx, q, ldq, s, lds, pow2, st));
    }
    if (cdiv(rows, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    const int kind = x_dtype == FP8Q_BF16 ? 1 : 0;
    return status_of(fp8q::launch_quantize_128x1(x, kind, rows, cols, ldx, nullptr, 0, q, ldq, s, lds, pow2, st));
}

int fp8q_quantize_act(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int tile,
                      uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
    return quantize_act_impl(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, FP8Q_SCALE_FP32, stream);
}

int fp8q_quantize_act_ex(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int tile,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds, int scale_mode, void* stream) {
    return quantize_act_impl(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, scale_mode, stream);
}

int fp8q_gather_quantize_act(const void* x, int x_dtype, int64_t rows_in, int64_t cols, int64_t ldx,
                             const int32_t* row_index, int64_t rows_out, uint8_t* q, int64_t ldq, float* s,
                             int64_t lds, int scale_mode, void* stream) {
    if (!valid_dtype(x_dtype) || !valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (rows_in < 0 || rows_out < 0 || cols < 0 || ldx < cols || ldq < cols || lds < rows_out) return FP8Q_ESHAPE;
    if (rows_out == 0 || cols == 0) return FP8Q_OK;
    if (!row_index || !q || !s || (rows_in > 0 && !x)) return FP8Q_EINVAL;
    const int eb = elem_bytes(x_dtype);
    if ((rows_in > 0 && !aligned(x, 16)) || (ldx * eb) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0 ||
        !aligned(s, 4) || !aligned(row_index, 4))
        return FP8Q_EALIGN;
    if (cdiv(cols, 512) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return status_of(fp8q::launch_gather_quantize_1x128(x, x_dtype, rows_in, cols, ldx, row_index, rows_out, q,
                                                        ldq, s, lds, scale_mode == FP8Q_SCALE_POW2,
                                                        static_cast<hipStream_t>(stream)));
}

static int quantize_weight_impl(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, float* s, int64_t lds, int scale_mode, void* stream) {
    if (!valid_dtype(w_dtype) || !valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (N < 0 || K < 0 || ldw < K || ldq < K || lds < cdiv(K, 128)) return FP8Q_ESHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_EINVAL;
    const int eb = elem_bytes(w_dtype);
    if (!aligned(w, 16) || (ldw * eb) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0 || !aligned(s, 4))
        return FP8Q_EALIGN;
    if (cdiv(N, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return status_of(fp8q::launch_quantize_128x128(w, w_dtype, N, K, ldw, q, ldq, s, lds,
                                                   scale_mode == FP8Q_SCALE_POW2,
                                                   static_cast<hipStream_t>(stream)));
}

int fp8q_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                         int64_t ldq, float* s, int64_t lds, void* stream) {
    return quantize_weight_impl(w, w_dtype, N, K, ldw, q, ldq, s, lds, FP8Q_SCALE_FP32, stream);
}

int fp8q_quantize_weight_ex(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                            int64_t ldq, float* s, int64_t lds, int scale_mode, void* stream) {
    return quantize_weight_impl(w, w_dtype, N, K, ldw, q, ldq, s, lds, scale_mode, stream);
}

static int requant_impl(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                        uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, int scale_mode, void* stream) {
    if (!valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (rows < 0 || cols < 0 || ldq < cols || lds < rows || ldqt < rows || ldst < cols) return FP8Q_ESHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!q || !s || !qt || !st) return FP8Q_EINVAL;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qt, 16) || ldqt % 16 != 0 || !aligned(s, 4) ||
        !aligned(st, 4))
        return FP8Q_EALIGN;
    if (cdiv(rows, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return status_of(fp8q::launch_quantize_128x1(q, 2, rows, cols, ldq, s, lds, qt, ldqt, st, ldst,
                                                 scale_mode == FP8Q_SCALE_POW2,
                                                 static_cast<hipStream_t>(stream)));
}

int fp8q_requant_transpose(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                           int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, void* stream) {
    return requant_impl(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, FP8Q_SCALE_FP32, stream);
}

int fp8q_requant_transpose_ex(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                              int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, int scale_mode,
                              void* stream) {
    return requant_impl(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, scale_mode, stream);
}

int fp8q_transpose_weight(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, const float* s, int64_t lds,
                          uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, void* stream) {
    if (N < 0 || K < 0 || ldq < K || ldqt < N || lds < cdiv(K, 128) || ldst < cdiv(N, 128)) return FP8Q_ESHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!q || !s || !qt || !st) return FP8Q_EINVAL;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qt, 16) || ldqt % 16 != 0 || !aligned(s, 4) ||
        !aligned(st, 4))
        return FP8Q_EALIGN;
    if (cdiv(N, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return status_of(fp8q::launch_transpose_weight(q, N, K, ldq, s, lds, qt, ldqt, st, ldst,
                                                   static_cast<hipStream_t>(stream)));
}

static int check_gemm_common(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* b,
                             int64_t ldb, const float* sb, int64_t M, int64_t N, int64_t K,
                             const void* c, int c_dtype, int64_t ldc) {
    if (!valid_dtype(c_dtype)) return FP8Q_EINVAL;
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8Q_ESHAPE;
    if (lda < K || ldb < K || ldc < N) return FP8Q_ESHAPE;
    // the kernels address a tile's rows with 32-bit byte offsets (256 rows)
    if (lda > kMaxOperandLd || ldb > kMaxOperandLd) return FP8Q_EUNSUPPORTED;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (K == 0) return FP8Q_ESHAPE;  // an empty contraction is not a GEMM this library runs
    if (!a || !sa || !b || !sb || !c) return FP8Q_EINVAL;
    if (!aligned(a, 16) || lda % 16 != 0 || !aligned(b, 16) || ldb % 16 != 0 || !aligned(sa, 4) ||
        !aligned(sb, 4) || !aligned(c, (uintptr_t)elem_bytes(c_dtype)))
        return FP8Q_EALIGN;
    return -1;  // proceed
}

static int gemm_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                     int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K,
                     void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags, void* stream,
                     void* workspace = nullptr, int64_t workspace_bytes = 0, bool validate_only = false) {
    if (bscale != FP8Q_BSCALE_BLOCK128 && bscale != FP8Q_BSCALE_ROW) return FP8Q_EINVAL;
    if ((flags & ~kKnownGemmFlags) != 0u) return FP8Q_EINVAL;
    if (accumulate && c_dtype != FP8Q_F32) return FP8Q_EUNSUPPORTED;
    const int rc = check_gemm_common(a, lda, sa, b, ldb, sb, M, N, K, c, c_dtype, ldc);
    if (rc >= 0) return rc;
    if (ldsa < M) return FP8Q_ESHAPE;
    if (bscale == FP8Q_BSCALE_BLOCK128 ? ldsb < K / 128 : ldsb < N) return FP8Q_ESHAPE;
    if (validate_only) return FP8Q_OK;
    fp8q::GemmArgs g{};
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.b_group_stride = 0;
    g.sb = sb; g.ldsb = ldsb; g.sb_group_stride = 0;
    g.offsets = nullptr; g.groups = 1;
    g.M = M; g.N = N; g.K = K; g.c = c; g.ldc = ldc;
    g.bscale = bscale; g.c_dtype = c_dtype; g.accumulate = accumulate ? 1 : 0;
    g.mma = datapath_of(flags);
    g.workspace = workspace;
    g.workspace_bytes = workspace_bytes;
    return status_of(fp8q::launch_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8q_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
              const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K, void* c,
              int c_dtype, int64_t ldc, int accumulate, void* stream) {
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, 0u,
                     stream);
}

int fp8q_gemm_ex(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                 int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K,
                 void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags, void* stream) {
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags,
                     stream);
}

int64_t fp8q_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) return 0;
    return fp8q::plan_splitk(M, N, K).bytes;
}

int fp8q_gemm_splitk(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                     int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K,
                     void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags, void* workspace,
                     int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return FP8Q_ESHAPE;
    const int64_t need = fp8q_gemm_splitk_workspace(M, N, K);
    if (need > 0) {
        if (!workspace) return FP8Q_EINVAL;
        if (workspace_bytes < need) return FP8Q_ESHAPE;
        if (!aligned(workspace, 256)) return FP8Q_EALIGN;
    }
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags,
                     stream, need > 0 ? workspace : nullptr, need);
}

int fp8q_gemm_splitk_noalloc(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                             int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N,
                             int64_t K, void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags,
                             void* stream) {
    const int64_t need = fp8q_gemm_splitk_workspace(M, N, K);
    if (need > (int64_t)FP8Q_SPLITK_SCRATCH_BYTES) return FP8Q_EUNSUPPORTED;
    void* ws = nullptr;
    if (need > 0) {
        // argument errors take precedence over the scratch lookup: validate
        // with a non-null stand-in first (nothing is launched on error)
        const int rc = gemm_impl(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                 accumulate, flags, nullptr, nullptr, 0, /*validate_only=*/true);
        if (rc != FP8Q_OK) return rc;
        ws = scratch_ptr();
        if (!ws) return FP8Q_EHIP;
    }
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags,
                     stream, ws, need);
}

int fp8q_clock_probe(uint64_t* out, int64_t ticks, void* stream) {
    if (!out) return FP8Q_EINVAL;
    if (!aligned(out, 8)) return FP8Q_EALIGN;
    if (ticks <= 0 || ticks > 100000000) return FP8Q_ESHAPE;
    return status_of(fp8q::launch_clock_probe(out, ticks, static_cast<hipStream_t>(stream)));
}

static int grouped_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                      int64_t ldb, int64_t b_group_stride, const float* sb, int64_t ldsb,
                      int64_t sb_group_stride, const int32_t* group_offsets, int G, int64_t M_total,
                      int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, unsigned flags, void* stream) {
    if ((flags & ~kKnownGemmFlags) != 0u) return FP8Q_EINVAL;
    if (G < 1 || G > kMaxGroups) return FP8Q_ESHAPE;
    const int rc = check_gemm_common(a, lda, sa, b, ldb, sb, M_total, N, K, c, c_dtype, ldc);
    if (rc >= 0) return rc;
    if (!group_offsets) return FP8Q_EINVAL;
    if (!aligned(group_offsets, 4)) return FP8Q_EALIGN;
    if (M_total > INT32_MAX) return FP8Q_EUNSUPPORTED;
    if (ldsa < M_total || ldsb < K / 128) return FP8Q_ESHAPE;
    if (b_group_stride < (N - 1) * ldb + K || sb_group_stride < (cdiv(N, 128) - 1) * ldsb + K / 128)
        return FP8Q_ESHAPE;
    if (b_group_stride % 16 != 0) return FP8Q_EALIGN;
    fp8q::GemmArgs g{};
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.b_group_stride = b_group_stride;
    g.sb = sb; g.ldsb = ldsb; g.sb_group_stride = sb_group_stride;
    g.offsets = group_offsets; g.groups = G;
    g.M = M_total; g.N = N; g.K = K; g.c = c; g.ldc = ldc;
    g.bscale = FP8Q_BSCALE_BLOCK128; g.c_dtype = c_dtype; g.accumulate = 0;
    g.mma = datapath_of(flags);
    return status_of(fp8q::launch_grouped_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8q_grouped_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                      int64_t ldb, int64_t b_group_stride, const float* sb, int64_t ldsb,
                      int64_t sb_group_stride, const int32_t* group_offsets, int G, int64_t M_total,
                      int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, void* stream) {
    return grouped_impl(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb, sb_group_stride, group_offsets, G,
                        M_total, N, K, c, c_dtype, ldc, 0u, stream);
}

int fp8q_grouped_gemm_ex(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                         int64_t ldb, int64_t b_group_stride, const float* sb, int64_t ldsb,
                         int64_t sb_group_stride, const int32_t* group_offsets, int G, int64_t M_total,
                         int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, unsigned flags,
                         void* stream) {
    return grouped_impl(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb, sb_group_stride, group_offsets, G,
                        M_total, N, K, c, c_dtype, ldc, flags, stream);
}

}  // extern "C"
