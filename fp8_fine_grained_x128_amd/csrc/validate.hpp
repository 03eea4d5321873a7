// validate.hpp -- host-side argument checks of the C ABI (include/fp8q.h).
//
// Plain C++ with no HIP dependency (so that it can also be built and run
// under the host sanitizers).  Every function returns kLaunch when the call
// is valid and has work to enqueue, FP8Q_OK when it is valid and empty
// (nothing is launched), or the fp8q_status error to return.  Nothing here
// dereferences a pointer: pointers are only tested for null and alignment.
#pragma once

#include <stdint.h>

#include "../../include/fp8q.h"

namespace fp8q {
namespace check {

constexpr int kLaunch = -1;

// Grid-dimension limit of the quantizer launches (y / x extents).
constexpr int64_t kMaxGridY = 65535;
constexpr int kMaxGroups = 1024;
// The GEMM reads a tile's operand rows through a buffer descriptor with 32-bit
// offsets and a 32-bit record count: 256 rows * ld must stay below 2^32.
constexpr int64_t kMaxOperandLd = (int64_t(1) << 24) - 1;
// Leading dimensions beyond 2^32 elements are refused before any size
// arithmetic, so that the products formed below (a leading dimension times
// an element size, a row count or a block count) stay far inside int64.
constexpr int64_t kMaxLd = int64_t(1) << 32;
// Expert strides of the grouped GEMM (elements); the kernels multiply them by
// an expert index below 1024.
constexpr int64_t kMaxGroupStride = int64_t(1) << 50;
constexpr unsigned kKnownGemmFlags = FP8Q_GEMM_MMA_FP8 | FP8Q_GEMM_POW2_SCALES;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int elem_bytes(int dtype) { return dtype == FP8Q_BF16 ? 2 : 4; }
inline bool valid_dtype(int d) { return d == FP8Q_F32 || d == FP8Q_BF16; }
inline bool valid_scale_mode(int m) { return m == FP8Q_SCALE_FP32 || m == FP8Q_SCALE_POW2; }
inline bool ld_ok(int64_t ld) { return ld >= 0 && ld <= kMaxLd; }

inline int quantize_act(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int tile,
                        const void* q, int64_t ldq, const void* s, int64_t lds, int scale_mode) {
    if (!valid_dtype(x_dtype) || (tile != FP8Q_TILE_1x128 && tile != FP8Q_TILE_128x1)) return FP8Q_EINVAL;
    if (!valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (rows < 0 || cols < 0 || !ld_ok(ldx) || !ld_ok(ldq) || !ld_ok(lds)) return FP8Q_ESHAPE;
    if (ldx < cols) return FP8Q_ESHAPE;
    if (tile == FP8Q_TILE_1x128) {
        if (ldq < cols || lds < rows) return FP8Q_ESHAPE;
    } else {
        if (ldq < rows || lds < cols) return FP8Q_ESHAPE;
    }
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_EINVAL;
    if (!aligned(x, 16) || (ldx * elem_bytes(x_dtype)) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0 ||
        !aligned(s, 4))
        return FP8Q_EALIGN;
    if (tile == FP8Q_TILE_1x128 ? cdiv(cols, 512) > kMaxGridY : cdiv(rows, 128) > kMaxGridY)
        return FP8Q_EUNSUPPORTED;
    return kLaunch;
}

inline int gather_quantize_act(const void* x, int x_dtype, int64_t rows_in, int64_t cols, int64_t ldx,
                               const void* row_index, int64_t rows_out, const void* q, int64_t ldq,
                               const void* s, int64_t lds, int scale_mode) {
    if (!valid_dtype(x_dtype) || !valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (!ld_ok(ldx) || !ld_ok(ldq) || !ld_ok(lds)) return FP8Q_ESHAPE;
    if (rows_in < 0 || rows_out < 0 || cols < 0 || ldx < cols || ldq < cols || lds < rows_out) return FP8Q_ESHAPE;
    if (rows_out == 0 || cols == 0) return FP8Q_OK;
    if (!row_index || !q || !s || (rows_in > 0 && !x)) return FP8Q_EINVAL;
    if ((rows_in > 0 && !aligned(x, 16)) || (ldx * elem_bytes(x_dtype)) % 16 != 0 || !aligned(q, 16) ||
        ldq % 16 != 0 || !aligned(s, 4) || !aligned(row_index, 4))
        return FP8Q_EALIGN;
    if (cdiv(cols, 512) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return kLaunch;
}

inline int quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw, const void* q,
                           int64_t ldq, const void* s, int64_t lds, int scale_mode) {
    if (!valid_dtype(w_dtype) || !valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (!ld_ok(ldw) || !ld_ok(ldq) || !ld_ok(lds)) return FP8Q_ESHAPE;
    if (N < 0 || K < 0 || ldw < K || ldq < K || lds < cdiv(K, 128)) return FP8Q_ESHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_EINVAL;
    if (!aligned(w, 16) || (ldw * elem_bytes(w_dtype)) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0 ||
        !aligned(s, 4))
        return FP8Q_EALIGN;
    if (cdiv(N, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return kLaunch;
}

inline int requant(const void* q, int64_t rows, int64_t cols, int64_t ldq, const void* s, int64_t lds,
                   const void* qt, int64_t ldqt, const void* st, int64_t ldst, int scale_mode) {
    if (!valid_scale_mode(scale_mode)) return FP8Q_EINVAL;
    if (!ld_ok(ldq) || !ld_ok(lds) || !ld_ok(ldqt) || !ld_ok(ldst)) return FP8Q_ESHAPE;
    if (rows < 0 || cols < 0 || ldq < cols || lds < rows || ldqt < rows || ldst < cols) return FP8Q_ESHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!q || !s || !qt || !st) return FP8Q_EINVAL;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qt, 16) || ldqt % 16 != 0 || !aligned(s, 4) ||
        !aligned(st, 4))
        return FP8Q_EALIGN;
    if (cdiv(rows, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return kLaunch;
}

inline int transpose_weight(const void* q, int64_t N, int64_t K, int64_t ldq, const void* s, int64_t lds,
                            const void* qt, int64_t ldqt, const void* st, int64_t ldst) {
    if (!ld_ok(ldq) || !ld_ok(lds) || !ld_ok(ldqt) || !ld_ok(ldst)) return FP8Q_ESHAPE;
    if (N < 0 || K < 0 || ldq < K || ldqt < N || lds < cdiv(K, 128) || ldst < cdiv(N, 128)) return FP8Q_ESHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!q || !s || !qt || !st) return FP8Q_EINVAL;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qt, 16) || ldqt % 16 != 0 || !aligned(s, 4) ||
        !aligned(st, 4))
        return FP8Q_EALIGN;
    if (cdiv(N, 128) > kMaxGridY) return FP8Q_EUNSUPPORTED;
    return kLaunch;
}

// Checks shared by the plain and the grouped GEMM.
inline int gemm_common(const void* a, int64_t lda, const void* sa, const void* b, int64_t ldb, const void* sb,
                       int64_t M, int64_t N, int64_t K, const void* c, int c_dtype, int64_t ldc, unsigned flags) {
    if (!valid_dtype(c_dtype) || (flags & ~kKnownGemmFlags) != 0u) return FP8Q_EINVAL;
    if (!ld_ok(lda) || !ld_ok(ldb) || !ld_ok(ldc)) return FP8Q_ESHAPE;
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8Q_ESHAPE;
    if (lda < K || ldb < K || ldc < N) return FP8Q_ESHAPE;
    if (lda > kMaxOperandLd || ldb > kMaxOperandLd) return FP8Q_EUNSUPPORTED;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (K == 0) return FP8Q_ESHAPE;  // an empty contraction is not a GEMM this library runs
    if (!a || !sa || !b || !sb || !c) return FP8Q_EINVAL;
    if (!aligned(a, 16) || lda % 16 != 0 || !aligned(b, 16) || ldb % 16 != 0 || !aligned(sa, 4) ||
        !aligned(sb, 4) || !aligned(c, (uintptr_t)elem_bytes(c_dtype)))
        return FP8Q_EALIGN;
    return kLaunch;
}

inline int gemm(const void* a, int64_t lda, const void* sa, int64_t ldsa, const void* b, int64_t ldb,
                const void* sb, int64_t ldsb, int bscale, int64_t M, int64_t N, int64_t K, const void* c,
                int c_dtype, int64_t ldc, int accumulate, unsigned flags) {
    if (bscale != FP8Q_BSCALE_BLOCK128 && bscale != FP8Q_BSCALE_ROW) return FP8Q_EINVAL;
    if ((flags & ~kKnownGemmFlags) != 0u) return FP8Q_EINVAL;
    if (accumulate && c_dtype != FP8Q_F32) return FP8Q_EUNSUPPORTED;
    const int rc = gemm_common(a, lda, sa, b, ldb, sb, M, N, K, c, c_dtype, ldc, flags);
    if (rc != kLaunch) return rc;
    if (ldsa < M) return FP8Q_ESHAPE;
    if (bscale == FP8Q_BSCALE_BLOCK128 ? ldsb < K / 128 : ldsb < N) return FP8Q_ESHAPE;
    return kLaunch;
}

// Split-K workspace (need: the plan's bytes, 0 when the shape does not split).
inline int splitk_workspace(int64_t need, const void* workspace, int64_t workspace_bytes) {
    if (workspace_bytes < 0) return FP8Q_ESHAPE;
    if (need > 0) {
        if (!workspace) return FP8Q_EINVAL;
        if (workspace_bytes < need) return FP8Q_ESHAPE;
        if (!aligned(workspace, 256)) return FP8Q_EALIGN;
    }
    return kLaunch;
}

inline int grouped(const void* a, int64_t lda, const void* sa, int64_t ldsa, const void* b, int64_t ldb,
                   int64_t b_group_stride, const void* sb, int64_t ldsb, int64_t sb_group_stride,
                   const void* group_offsets, int G, int64_t M_total, int64_t N, int64_t K, const void* c,
                   int c_dtype, int64_t ldc, unsigned flags) {
    if ((flags & ~kKnownGemmFlags) != 0u) return FP8Q_EINVAL;
    if (G < 1 || G > kMaxGroups) return FP8Q_ESHAPE;
    const int rc = gemm_common(a, lda, sa, b, ldb, sb, M_total, N, K, c, c_dtype, ldc, flags);
    if (rc != kLaunch) return rc;
    if (!group_offsets) return FP8Q_EINVAL;
    if (!aligned(group_offsets, 4)) return FP8Q_EALIGN;
    if (M_total > INT32_MAX) return FP8Q_EUNSUPPORTED;
    if (!ld_ok(ldsa) || !ld_ok(ldsb) || b_group_stride < 0 || b_group_stride > kMaxGroupStride ||
        sb_group_stride < 0 || sb_group_stride > kMaxGroupStride)
        return FP8Q_ESHAPE;
    if (ldsa < M_total || ldsb < K / 128) return FP8Q_ESHAPE;
    // N <= ldc <= 2^32 and ldb < 2^24, ldsb <= 2^32: both products stay below 2^57
    if (b_group_stride < (N - 1) * ldb + K || sb_group_stride < (cdiv(N, 128) - 1) * ldsb + K / 128)
        return FP8Q_ESHAPE;
    if (b_group_stride % 16 != 0) return FP8Q_EALIGN;
    return kLaunch;
}

inline int clock_probe(const void* out, int64_t ticks) {
    if (!out) return FP8Q_EINVAL;
    if (!aligned(out, 8)) return FP8Q_EALIGN;
    if (ticks <= 0 || ticks > 100000000) return FP8Q_ESHAPE;
    return kLaunch;
}

}  // namespace check
}  // namespace fp8q
