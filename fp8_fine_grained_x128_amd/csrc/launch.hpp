// launch.hpp -- internal launcher declarations shared by the kernel sources
// and the C ABI layer.  Not part of the public interface (include/fp8q.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int kDtypeF32 = 0;   // FP8Q_F32
constexpr int kDtypeBF16 = 1;  // FP8Q_BF16

// pow2: 0 fp32 scales fl32(amax/448), 1 power-of-two scales
hipError_t launch_quantize_1x128(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, int pow2, hipStream_t st);

// Row gather (row_index on the device, [rows_out]) fused with the 1x128 quantizer.
hipError_t launch_gather_quantize_1x128(const void* x, int dtype, int64_t rows_in, int64_t cols, int64_t ldx,
                                        const int32_t* row_index, int64_t rows_out, uint8_t* q, int64_t ldq,
                                        float* s, int64_t lds, int pow2, hipStream_t st);

hipError_t launch_quantize_128x128(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds, int pow2, hipStream_t st);

// kind: 0 fp32 input, 1 bf16 input, 2 cached fp8 codes + 1x128 scales (s_in)
hipError_t launch_quantize_128x1(const void* x, int kind, int64_t rows, int64_t cols, int64_t ldx,
                                 const float* s_in, int64_t lds_in, uint8_t* qt, int64_t ldqt,
                                 float* st_out, int64_t ldst, int pow2, hipStream_t st);

hipError_t launch_transpose_weight(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, const float* s,
                                   int64_t lds, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                                   hipStream_t stream);

struct GemmArgs {
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    int64_t b_group_stride;
    const float* sb;
    int64_t ldsb;
    int64_t sb_group_stride;
    const int32_t* offsets;  // grouped only
    int groups;              // grouped only
    int64_t M, N, K;
    void* c;
    int64_t ldc;
    int bscale;      // 0 block128, 1 row
    int c_dtype;     // kDtypeF32 / kDtypeBF16
    int accumulate;  // fp32 only
    int mma;         // matrix-core datapath (kMma*)
    void* workspace;          // split-K partials (plain GEMM only; nullptr: no split)
    int64_t workspace_bytes;
};

constexpr int kMmaF16 = 0;        // f16 MFMA on exactly converted codes, promotion per chunk
constexpr int kMmaFp8 = 1;        // native FP8 MFMA per chunk, promotion per chunk
constexpr int kMmaBf16Fold = 2;   // power-of-two scales folded into exact bf16 operands, no promotion
constexpr int kMmaFp8Scaled = 3;  // block-scaled FP8 MFMA with E8M0 operand scales, no promotion

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

// Shader-clock probe (measurement support): out[0] real-time ticks,
// out[1] shader-clock cycles, out[2] real-time counter rate in kHz.
hipError_t launch_clock_probe(uint64_t* out, int64_t ticks, hipStream_t st);

// Split-K plan of the plain GEMM: slices (1 = no split), chunks per slice and
// the workspace bytes the slices' FP32 partials take ([slices][M][ldws],
// ldws = N rounded up to a multiple of 4).
struct SplitPlan {
    int slices;
    int64_t kb_split;
    int64_t ldws;
    int64_t bytes;
};
SplitPlan plan_splitk(int64_t M, int64_t N, int64_t K);
hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t st);

}  // namespace fp8q
