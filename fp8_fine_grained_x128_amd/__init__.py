"""fp8q: fine-grained FP8 linear-layer kernels for AMD Instinct MI355X (gfx950).

Importing the package loads the in-tree HIP library ``libfp8q.so``; the
computation entry points are in :mod:`.binding`.  Synthetic workloads live in
:mod:`.workloads` (importable without the library).
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    EXPORTS, FP8Q_BF16, FP8Q_BSCALE_BLOCK128, FP8Q_BSCALE_ROW, FP8Q_EALIGN, FP8Q_EHIP, FP8Q_EINVAL,
    FP8Q_ESHAPE, FP8Q_EUNSUPPORTED, FP8Q_F32, FP8Q_GEMM_MMA_FP8, FP8Q_GEMM_POW2_SCALES, FP8Q_OK, FP8Q_SCALE_FP32,
    FP8Q_SCALE_POW2, FP8Q_TILE_128x1, FP8Q_TILE_1x128, Fp8qError, LIB_PATH, fp8q_gemm, fp8q_gemm_ex,
    fp8q_grouped_gemm, fp8q_grouped_gemm_ex, fp8q_quantize_act, fp8q_quantize_act_ex,
    fp8q_quantize_weight, fp8q_quantize_weight_ex, fp8q_requant_transpose,
    fp8q_requant_transpose_ex, fp8q_strerror, fp8q_version, gemm, grouped_gemm, library,
    quantize_act, quantize_weight, requant_transpose, transpose_weight, dgrad,
    fp8q_transpose_weight, fp8q_gather_quantize_act, gather_quantize_act, fp8q_gemm_splitk, fp8q_clock_probe,
    fp8q_gemm_splitk_noalloc, SPLITK_SCRATCH_BYTES,
    fp8q_gemm_splitk_workspace,
)

__version__ = "0.2.0"
