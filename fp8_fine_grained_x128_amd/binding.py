"""ctypes binding of libfp8q.so (the C ABI in include/fp8q.h).

Two layers, both argument marshalling only:

* ``fp8q_*`` functions with the C names and C argument lists (device pointers
  as Python ints, ``stream`` as an int handle or None);
* tensor helpers (``quantize_act``, ``quantize_weight``, ``requant_transpose``,
  ``gemm``, ``grouped_gemm``) that take torch tensors on the HIP device,
  allocate outputs with torch, derive leading dimensions from strides and
  enqueue on torch's current stream.

Every computation runs in the library's HIP kernels.  If the library is not
built, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

FP8Q_OK = 0
FP8Q_EINVAL = 1
FP8Q_ESHAPE = 2
FP8Q_EALIGN = 3
FP8Q_EUNSUPPORTED = 4
FP8Q_EHIP = 5

FP8Q_F32 = 0
FP8Q_BF16 = 1
FP8Q_TILE_1x128 = 0
FP8Q_TILE_128x1 = 1
FP8Q_BSCALE_BLOCK128 = 0
FP8Q_BSCALE_ROW = 1
FP8Q_GEMM_MMA_FP8 = 1
FP8Q_GEMM_POW2_SCALES = 2
FP8Q_SCALE_FP32 = 0
FP8Q_SCALE_POW2 = 1

EXPORTS = ("fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_requant_transpose", "fp8q_gemm",
           "fp8q_grouped_gemm", "fp8q_gemm_ex", "fp8q_grouped_gemm_ex", "fp8q_quantize_act_ex",
           "fp8q_quantize_weight_ex", "fp8q_requant_transpose_ex", "fp8q_transpose_weight",
           "fp8q_gather_quantize_act", "fp8q_gemm_splitk", "fp8q_gemm_splitk_noalloc", "fp8q_clock_probe",
           "fp8q_gemm_splitk_workspace", "fp8q_strerror", "fp8q_version")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int

_lib.fp8q_quantize_act.argtypes = [_p, _i32, _i64, _i64, _i64, _i32, _p, _i64, _p, _i64, _p]
_lib.fp8q_quantize_weight.argtypes = [_p, _i32, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]
_lib.fp8q_requant_transpose.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.fp8q_gemm.argtypes = [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i32, _i64, _i64, _i64, _p, _i32,
                           _i64, _i32, _p]
_lib.fp8q_grouped_gemm.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i32, _i64,
                                   _i64, _i64, _p, _i32, _i64, _p]
_u32 = ctypes.c_uint
_lib.fp8q_gemm_ex.argtypes = _lib.fp8q_gemm.argtypes[:-1] + [_u32, _p]
_lib.fp8q_grouped_gemm_ex.argtypes = _lib.fp8q_grouped_gemm.argtypes[:-1] + [_u32, _p]
_lib.fp8q_quantize_act_ex.argtypes = _lib.fp8q_quantize_act.argtypes[:-1] + [_i32, _p]
_lib.fp8q_quantize_weight_ex.argtypes = _lib.fp8q_quantize_weight.argtypes[:-1] + [_i32, _p]
_lib.fp8q_requant_transpose_ex.argtypes = _lib.fp8q_requant_transpose.argtypes[:-1] + [_i32, _p]
_lib.fp8q_transpose_weight.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.fp8q_gather_quantize_act.argtypes = [_p, _i32, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i32, _p]
_lib.fp8q_gemm_splitk.argtypes = _lib.fp8q_gemm.argtypes[:-1] + [_u32, _p, _i64, _p]
_lib.fp8q_gemm_splitk_noalloc.argtypes = _lib.fp8q_gemm.argtypes[:-1] + [_u32, _p]
_lib.fp8q_clock_probe.argtypes = [_p, _i64, _p]
_lib.fp8q_gemm_splitk_workspace.argtypes = [_i64, _i64, _i64]
_lib.fp8q_gemm_splitk_workspace.restype = _i64
_lib.fp8q_strerror.argtypes = [_i32]
_lib.fp8q_strerror.restype = ctypes.c_char_p
_lib.fp8q_version.argtypes = []
for _n in EXPORTS[:-3]:
    getattr(_lib, _n).restype = _i32


def library() -> ctypes.CDLL:
    return _lib


# ------------------------------------------------------------------ C names

def fp8q_quantize_act(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, stream=None) -> int:
    return _lib.fp8q_quantize_act(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, stream)


def fp8q_quantize_weight(w, w_dtype, N, K, ldw, q, ldq, s, lds, stream=None) -> int:
    return _lib.fp8q_quantize_weight(w, w_dtype, N, K, ldw, q, ldq, s, lds, stream)


def fp8q_requant_transpose(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, stream=None) -> int:
    return _lib.fp8q_requant_transpose(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, stream)


def fp8q_gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate,
              stream=None) -> int:
    return _lib.fp8q_gemm(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                          accumulate, stream)


def fp8q_grouped_gemm(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb, sb_group_stride,
                      group_offsets, G, M_total, N, K, c, c_dtype, ldc, stream=None) -> int:
    return _lib.fp8q_grouped_gemm(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb,
                                  sb_group_stride, group_offsets, G, M_total, N, K, c, c_dtype, ldc,
                                  stream)


def fp8q_quantize_act_ex(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, scale_mode,
                         stream=None) -> int:
    return _lib.fp8q_quantize_act_ex(x, x_dtype, rows, cols, ldx, tile, q, ldq, s, lds, scale_mode,
                                     stream)


def fp8q_quantize_weight_ex(w, w_dtype, N, K, ldw, q, ldq, s, lds, scale_mode, stream=None) -> int:
    return _lib.fp8q_quantize_weight_ex(w, w_dtype, N, K, ldw, q, ldq, s, lds, scale_mode, stream)


def fp8q_requant_transpose_ex(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, scale_mode,
                              stream=None) -> int:
    return _lib.fp8q_requant_transpose_ex(q, rows, cols, ldq, s, lds, qt, ldqt, st, ldst, scale_mode,
                                          stream)


def fp8q_transpose_weight(q, N, K, ldq, s, lds, qt, ldqt, st, ldst, stream=None) -> int:
    return _lib.fp8q_transpose_weight(q, N, K, ldq, s, lds, qt, ldqt, st, ldst, stream)


def fp8q_gather_quantize_act(x, x_dtype, rows_in, cols, ldx, row_index, rows_out, q, ldq, s, lds,
                             scale_mode, stream=None) -> int:
    return _lib.fp8q_gather_quantize_act(x, x_dtype, rows_in, cols, ldx, row_index, rows_out, q, ldq, s,
                                         lds, scale_mode, stream)


def fp8q_gemm_ex(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate,
                 flags, stream=None) -> int:
    return _lib.fp8q_gemm_ex(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                             accumulate, flags, stream)


def fp8q_grouped_gemm_ex(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb, sb_group_stride,
                         group_offsets, G, M_total, N, K, c, c_dtype, ldc, flags, stream=None) -> int:
    return _lib.fp8q_grouped_gemm_ex(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, ldsb,
                                     sb_group_stride, group_offsets, G, M_total, N, K, c, c_dtype,
                                     ldc, flags, stream)


def fp8q_gemm_splitk(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate,
                     flags, workspace, workspace_bytes, stream=None) -> int:
    return _lib.fp8q_gemm_splitk(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                 accumulate, flags, workspace, workspace_bytes, stream)


def fp8q_gemm_splitk_noalloc(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc, accumulate,
                             flags, stream=None) -> int:
    return _lib.fp8q_gemm_splitk_noalloc(a, lda, sa, ldsa, b, ldb, sb, ldsb, bscale, M, N, K, c, c_dtype, ldc,
                                         accumulate, flags, stream)


SPLITK_SCRATCH_BYTES = 64 << 20


def fp8q_clock_probe(out, ticks, stream=None) -> int:
    return _lib.fp8q_clock_probe(out, ticks, stream)


def fp8q_gemm_splitk_workspace(M, N, K) -> int:
    return _lib.fp8q_gemm_splitk_workspace(M, N, K)


def fp8q_strerror(status: int) -> str:
    return _lib.fp8q_strerror(status).decode()


def fp8q_version() -> int:
    return _lib.fp8q_version()


# ------------------------------------------------------------------ helpers

class Fp8qError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fp8q_strerror(status)} (status {status})")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != FP8Q_OK:
        raise Fp8qError(status, what)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP8Q_F32
    if t.dtype == torch.bfloat16:
        return FP8Q_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    """Row stride in elements.  A single-row tensor may carry any stride (its
    row stride never multiplies a nonzero index), so report the smallest value
    that satisfies the library's 16-byte rule for that dtype."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    if t.shape[0] <= 1:
        per16 = max(1, 16 // t.element_size())
        return max(per16, -(-t.shape[1] // per16) * per16)
    return t.stride(0)


def _on_device(what: str, *ts: torch.Tensor) -> None:
    """Every tensor on the same HIP device (a host tensor's data_ptr would be
    handed to a kernel)."""
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError(f"{what}: tensors must be on a HIP device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensors on different devices ({dev}, {t.device})")


def _check_codes(what: str, t: torch.Tensor) -> None:
    if t.element_size() != 1 or t.is_floating_point():
        raise ValueError(f"{what}: codes must be a 1-byte integer tensor (uint8 E4M3 bytes), got {t.dtype}")


def _check_scales(what: str, t: torch.Tensor, rows: int, cols: int) -> None:
    """float32 scales, 2-D, at least rows x cols with unit column stride."""
    if t.dtype != torch.float32:
        raise ValueError(f"{what}: scales must be float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{what}: scales of shape {tuple(t.shape)} do not hold [{rows}][{cols}]")


def _pad16(n: int) -> int:
    return (n + 15) // 16 * 16


def _codes(rows: int, cols: int, device) -> torch.Tensor:
    """uint8 [rows][cols] with a 16-byte-multiple row stride."""
    buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.uint8, device=device)
    return buf[:, :cols]


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def quantize_act(x: torch.Tensor, tile: int = FP8Q_TILE_1x128,
                 scale_mode: int = FP8Q_SCALE_FP32) -> Tuple[torch.Tensor, torch.Tensor]:
    """1x128: returns codes [rows][cols] and scales [ceil(cols/128)][rows].
    128x1: returns codes [cols][rows] (transposed) and scales [ceil(rows/128)][cols]."""
    _on_device("quantize_act", x)
    rows, cols = x.shape
    if tile == FP8Q_TILE_1x128:
        q = _codes(rows, cols, x.device)
        s = torch.empty((_cdiv(cols, 128), rows), dtype=torch.float32, device=x.device)
    else:
        q = _codes(cols, rows, x.device)
        s = torch.empty((_cdiv(rows, 128), cols), dtype=torch.float32, device=x.device)
    args = (x.data_ptr(), _dtype_code(x), rows, cols, _ld(x), tile, q.data_ptr(), _ld(q), s.data_ptr(),
            max(s.stride(0), 1))
    if scale_mode == FP8Q_SCALE_FP32:
        _check(fp8q_quantize_act(*args, _stream()), "fp8q_quantize_act")
    else:
        _check(fp8q_quantize_act_ex(*args, scale_mode, _stream()), "fp8q_quantize_act_ex")
    return q, s


def gather_quantize_act(x: torch.Tensor, row_index: torch.Tensor,
                        scale_mode: int = FP8Q_SCALE_FP32) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rows x[row_index[i]] quantized per 1x128 tile (an out-of-range index
    gives a zero row).  row_index: int32 on the device.  Returns codes
    [len][cols] and scales [ceil(cols/128)][len]."""
    if row_index.dtype != torch.int32 or row_index.dim() != 1 or not row_index.is_contiguous():
        raise ValueError("row_index must be a contiguous 1-D int32 tensor")
    _on_device("gather_quantize_act", x, row_index)
    rows_in, cols = x.shape
    rows_out = row_index.numel()
    q = _codes(rows_out, cols, x.device)
    s = torch.empty((_cdiv(cols, 128), rows_out), dtype=torch.float32, device=x.device)
    _check(fp8q_gather_quantize_act(x.data_ptr(), _dtype_code(x), rows_in, cols, _ld(x), row_index.data_ptr(),
                                    rows_out, q.data_ptr(), _ld(q), s.data_ptr(), max(s.stride(0), 1),
                                    scale_mode, _stream()),
           "fp8q_gather_quantize_act")
    return q, s


def quantize_weight(w: torch.Tensor, scale_mode: int = FP8Q_SCALE_FP32) -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns codes [N][K] and 128x128 block scales [ceil(N/128)][ceil(K/128)]."""
    _on_device("quantize_weight", w)
    N, K = w.shape
    q = _codes(N, K, w.device)
    s = torch.empty((_cdiv(N, 128), _cdiv(K, 128)), dtype=torch.float32, device=w.device)
    args = (w.data_ptr(), _dtype_code(w), N, K, _ld(w), q.data_ptr(), _ld(q), s.data_ptr(),
            max(s.stride(0), 1))
    if scale_mode == FP8Q_SCALE_FP32:
        _check(fp8q_quantize_weight(*args, _stream()), "fp8q_quantize_weight")
    else:
        _check(fp8q_quantize_weight_ex(*args, scale_mode, _stream()), "fp8q_quantize_weight_ex")
    return q, s


def requant_transpose(q: torch.Tensor, s: torch.Tensor,
                      scale_mode: int = FP8Q_SCALE_FP32) -> Tuple[torch.Tensor, torch.Tensor]:
    """Cached 1x128 codes q[rows][cols] + scales s[ceil(cols/128)][rows] ->
    128x1 codes qt[cols][rows] + scales st[ceil(rows/128)][cols]."""
    _check_codes("requant_transpose codes", q)
    rows, cols = q.shape
    _check_scales("requant_transpose scales (layout [ceil(cols/128)][rows])", s, _cdiv(cols, 128), rows)
    _on_device("requant_transpose", q, s)
    qt = _codes(cols, rows, q.device)
    st = torch.empty((_cdiv(rows, 128), cols), dtype=torch.float32, device=q.device)
    args = (q.data_ptr(), rows, cols, _ld(q), s.data_ptr(), _ld(s), qt.data_ptr(), _ld(qt), st.data_ptr(),
            max(st.stride(0), 1))
    if scale_mode == FP8Q_SCALE_FP32:
        _check(fp8q_requant_transpose(*args, _stream()), "fp8q_requant_transpose")
    else:
        _check(fp8q_requant_transpose_ex(*args, scale_mode, _stream()), "fp8q_requant_transpose_ex")
    return qt, st


def transpose_weight(q: torch.Tensor, s: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Cached weight codes q[N][K] + block scales s[ceil(N/128)][ceil(K/128)] ->
    qt[K][N] + st[ceil(K/128)][ceil(N/128)] (the Dgrad operand, exact)."""
    _check_codes("transpose_weight codes", q)
    N, K = q.shape
    _check_scales("transpose_weight scales (layout [ceil(N/128)][ceil(K/128)])", s, _cdiv(N, 128), _cdiv(K, 128))
    _on_device("transpose_weight", q, s)
    qt = _codes(K, N, q.device)
    st = torch.empty((_cdiv(K, 128), _cdiv(N, 128)), dtype=torch.float32, device=q.device)
    _check(fp8q_transpose_weight(q.data_ptr(), N, K, _ld(q), s.data_ptr(), _ld(s), qt.data_ptr(), _ld(qt),
                                 st.data_ptr(), _ld(st), _stream()),
           "fp8q_transpose_weight")
    return qt, st


def dgrad(dy_q: torch.Tensor, dy_s: torch.Tensor, wt_q: torch.Tensor, wt_s: torch.Tensor,
          out_dtype: torch.dtype = torch.bfloat16, flags: int = 0) -> torch.Tensor:
    """dX[M][K] = dY[M][N] W[N][K] from dY's 1x128 codes/scales and the
    transposed weight of transpose_weight()."""
    return gemm(dy_q, dy_s, wt_q, wt_s, bscale=FP8Q_BSCALE_BLOCK128, out_dtype=out_dtype, flags=flags)


def gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
         bscale: int = FP8Q_BSCALE_BLOCK128, out_dtype: torch.dtype = torch.bfloat16,
         c: Optional[torch.Tensor] = None, accumulate: bool = False, flags: int = 0,
         split_k: bool = True) -> torch.Tensor:
    """C[M][N] = block-scaled A[M][K] . B[N][K]^T (see fp8q_gemm; `flags`
    selects the matrix-core datapath, see fp8q_gemm_ex).  With split_k, shapes
    that leave the GPU mostly idle run through fp8q_gemm_splitk with a
    workspace allocated here."""
    M, K = a.shape
    N = b.shape[0]
    if b.dim() != 2 or b.shape[1] != K:
        raise ValueError(f"gemm: A is [{M}][{K}] but B is {tuple(b.shape)}; B must be [N][{K}]")
    _check_codes("gemm A", a)
    _check_codes("gemm B", b)
    _check_scales("gemm s_a (layout [K/128][M])", sa, K // 128, M)
    if bscale == FP8Q_BSCALE_BLOCK128:
        _check_scales("gemm s_b (BLOCK128 layout [ceil(N/128)][K/128])", sb, _cdiv(N, 128), K // 128)
    else:
        _check_scales("gemm s_b (ROW layout [K/128][N])", sb, K // 128, N)
    _on_device("gemm", a, sa, b, sb, *(() if c is None else (c,)))
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    elif c.dim() != 2 or tuple(c.shape) != (M, N):
        raise ValueError(f"gemm: C is {tuple(c.shape)}, expected [{M}][{N}]")
    args = (a.data_ptr(), _ld(a), sa.data_ptr(), _ld(sa), b.data_ptr(), _ld(b), sb.data_ptr(), _ld(sb),
            bscale, M, N, K, c.data_ptr(), _dtype_code(c), _ld(c), 1 if accumulate else 0)
    need = fp8q_gemm_splitk_workspace(M, N, K) if split_k else 0
    if need > 0:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=a.device)
        base = (ws.data_ptr() + 255) // 256 * 256
        _check(fp8q_gemm_splitk(*args, flags, base, need, _stream()), "fp8q_gemm_splitk")
    elif flags:
        _check(fp8q_gemm_ex(*args, flags, _stream()), "fp8q_gemm_ex")
    else:
        _check(fp8q_gemm(*args, _stream()), "fp8q_gemm")
    return c


def grouped_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                 offsets: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                 c: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """Per-expert block-scaled GEMM.  a [M_total][K] grouped by expert,
    b [G][N][K] codes, sb [G][ceil(N/128)][K/128], offsets int32 [G+1] on device."""
    M, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or offsets.dtype != torch.int32 or offsets.numel() != G + 1:
        raise ValueError("grouped_gemm: shape mismatch")
    if b.stride(2) != 1 or sb.stride(2) != 1:
        raise ValueError("grouped_gemm: unit inner stride required")
    _check_codes("grouped_gemm A", a)
    _check_codes("grouped_gemm B", b)
    _check_scales("grouped_gemm s_a (layout [K/128][M_total])", sa, K // 128, M)
    if sb.dtype != torch.float32 or sb.dim() != 3 or sb.shape[0] != G or sb.shape[1] < _cdiv(N, 128) \
            or sb.shape[2] < K // 128:
        raise ValueError(f"grouped_gemm: s_b {tuple(sb.shape)} {sb.dtype}, expected float32 "
                         f"[{G}][{_cdiv(N, 128)}][{K // 128}]")
    _on_device("grouped_gemm", a, sa, b, sb, offsets, *(() if c is None else (c,)))
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    args = (a.data_ptr(), _ld(a), sa.data_ptr(), _ld(sa), b.data_ptr(), b.stride(1), b.stride(0),
            sb.data_ptr(), sb.stride(1), sb.stride(0), offsets.data_ptr(), G, M, N, K, c.data_ptr(),
            _dtype_code(c), _ld(c))
    if flags:
        _check(fp8q_grouped_gemm_ex(*args, flags, _stream()), "fp8q_grouped_gemm_ex")
    else:
        _check(fp8q_grouped_gemm(*args, _stream()), "fp8q_grouped_gemm")
    return c
