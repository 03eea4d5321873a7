// fp8q_api.hip -- C ABI (include/fp8q.h): host-side validation
// (validate.hpp), then the kernel launches on the caller's stream.  No
// allocation, no synchronization; the only state is the per-device address
// of the split-K scratch array below, looked up once per device.
#include <stdint.h>

#include <mutex>

#include "../../include/fp8q.h"
#include "launch.hpp"
#include "validate.hpp"

// Device scratch of fp8q_gemm_splitk_noalloc: the split-K partials live here
// instead of in a caller workspace.  Each device that runs the library holds
// its own copy until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[FP8Q_SPLITK_SCRATCH_BYTES];

namespace {

using fp8q::check::kLaunch;

inline int status_of(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_EHIP; }

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

inline int datapath_of(unsigned flags) {
    const bool fp8 = (flags & FP8Q_GEMM_MMA_FP8) != 0u;
    if (flags & FP8Q_GEMM_POW2_SCALES) return fp8 ? fp8q::kMmaFp8Scaled : fp8q::kMmaBf16Fold;
    return fp8 ? fp8q::kMmaFp8 : fp8q::kMmaF16;
}

int quantize_act_impl(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int tile, uint8_t* q,
                      int64_t ldq, float* s, int64_t lds, int scale_mode, void* stream) {
    const int rc = fp8q::check::quantize_act(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, scale_mode);
    if (rc != kLaunch) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int pow2 = scale_mode == FP8Q_SCALE_POW2;
    if (tile == FP8Q_TILE_1x128)
        return status_of(fp8q::launch_quantize_1x128(x, x_dtype, rows, cols, ldx, q, ldq, s, lds, pow2, st));
    const int kind = x_dtype == FP8Q_BF16 ? 1 : 0;
    return status_of(fp8q::launch_quantize_128x1(x, kind, rows, cols, ldx, nullptr, 0, q, ldq, s, lds, pow2, st));
}

int quantize_weight_impl(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                         float* s, int64_t lds, int scale_mode, void* stream) {
    const int rc = fp8q::check::quantize_weight(w, w_dtype, N, K, ldw, q, ldq, s, lds, scale_mode);
    if (rc != kLaunch) return rc;
    return status_of(fp8q::launch_quantize_128x128(w, w_dtype, N, K, ldw, q, ldq, s, lds,
                                                   scale_mode == FP8Q_SCALE_POW2, static_cast<hipStream_t>(stream)));
}

int requant_impl(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                 uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, int scale_mode, void* stream) {
    const int rc = fp8q::check::requant(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, scale_mode);
    if (rc != kLaunch) return rc;
    return status_of(fp8q::launch_quantize_128x1(q, 2, rows, cols, ldq, s, lds, qt, ldqt, st, ldst,
                                                 scale_mode == FP8Q_SCALE_POW2, static_cast<hipStream_t>(stream)));
}

// The plain GEMM after validation; `workspace` holds the split-K partials
// when the shape splits (nullptr: no split).
int gemm_launch(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K, void* c, int c_dtype,
                int64_t ldc, int accumulate, unsigned flags, void* workspace, int64_t workspace_bytes,
                void* stream) {
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

int grouped_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
                 int64_t b_group_stride, const float* sb, int64_t ldsb, int64_t sb_group_stride,
                 const int32_t* group_offsets, int G, int64_t M_total, int64_t N, int64_t K, void* c,
                 int c_dtype, int64_t ldc, unsigned flags, void* stream) {
    const int rc = fp8q::check::grouped(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb, sb_group_stride,
                                        group_offsets, G, M_total, N, K, c, c_dtype, ldc, flags);
    if (rc != kLaunch) return rc;
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
    const int rc = fp8q::check::gather_quantize_act(x, x_dtype, rows_in, cols, ldx, row_index, rows_out, q, ldq,
                                                    s, lds, scale_mode);
    if (rc != kLaunch) return rc;
    return status_of(fp8q::launch_gather_quantize_1x128(x, x_dtype, rows_in, cols, ldx, row_index, rows_out, q,
                                                        ldq, s, lds, scale_mode == FP8Q_SCALE_POW2,
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
    const int rc = fp8q::check::transpose_weight(q, N, K, ldq, s, lds, qt, ldqt, st, ldst);
    if (rc != kLaunch) return rc;
    return status_of(fp8q::launch_transpose_weight(q, N, K, ldq, s, lds, qt, ldqt, st, ldst,
                                                   static_cast<hipStream_t>(stream)));
}

int fp8q_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b, int64_t ldb,
              const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K, void* c,
              int c_dtype, int64_t ldc, int accumulate, void* stream) {
    const int rc = fp8q::check::gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                     accumulate, 0u);
    if (rc != kLaunch) return rc;
    return gemm_launch(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, 0u,
                       nullptr, 0, stream);
}

int fp8q_gemm_ex(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                 int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K,
                 void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags, void* stream) {
    const int rc = fp8q::check::gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                     accumulate, flags);
    if (rc != kLaunch) return rc;
    return gemm_launch(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags,
                       nullptr, 0, stream);
}

int64_t fp8q_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) return 0;
    return fp8q::plan_splitk(M, N, K).bytes;
}

int fp8q_gemm_splitk(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                     int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K,
                     void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags, void* workspace,
                     int64_t workspace_bytes, void* stream) {
    const int64_t need = fp8q_gemm_splitk_workspace(M, N, K);
    int rc = fp8q::check::splitk_workspace(need, workspace, workspace_bytes);
    if (rc != kLaunch) return rc;
    rc = fp8q::check::gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate,
                           flags);
    if (rc != kLaunch) return rc;
    return gemm_launch(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags,
                       need > 0 ? workspace : nullptr, need, stream);
}

int fp8q_gemm_splitk_noalloc(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                             int64_t ldb, const float* sb, int64_t ldsb, int bscale, int64_t M, int64_t N,
                             int64_t K, void* c, int c_dtype, int64_t ldc, int accumulate, unsigned flags,
                             void* stream) {
    const int rc = fp8q::check::gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                     accumulate, flags);
    if (rc != kLaunch) return rc;
    const int64_t need = fp8q_gemm_splitk_workspace(M, N, K);
    if (need > (int64_t)FP8Q_SPLITK_SCRATCH_BYTES) return FP8Q_EUNSUPPORTED;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws) return FP8Q_EHIP;
    }
    return gemm_launch(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate, flags, ws,
                       need, stream);
}

int fp8q_clock_probe(uint64_t* out, int64_t ticks, void* stream) {
    const int rc = fp8q::check::clock_probe(out, ticks);
    if (rc != kLaunch) return rc;
    return status_of(fp8q::launch_clock_probe(out, ticks, static_cast<hipStream_t>(stream)));
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
