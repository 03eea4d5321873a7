"""CPU oracle for the fine-grained FP8 linear-layer path (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
this package.  The product library never imports, links or calls it; it shares
no code with the HIP kernels.

The arithmetic lives in ``fp8q_oracle.c`` (plain C, fp32/fp64, OpenMP).  This
module only loads the shared library built from it and marshals numpy arrays.
Layouts here are the "natural" ones (codes in the input's orientation, scales
indexed ``[tile_row][tile_col]``); tests map them to the library's layouts.

Sources are the five reference web pages, cited by site and post id; see the
header of ``fp8q_oracle.c`` for what each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# No fast-math and no FMA contraction: each fp32 / fp64 operation rounds once.
CFLAGS = ["-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra", "-Werror"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_native(out_dir: str) -> str:
    """Compile the same source with ``-march=native`` into ``out_dir`` (for
    timing the oracle on the host that runs it; the arithmetic is unchanged:
    no fast-math and no contraction, so every operation still rounds once).
    The in-tree library stays portable because it travels between hosts."""
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "liboracle_native.so")
    subprocess.run(["gcc", *CFLAGS, "-march=native", _SRC, "-o", path, "-lm"], check=True)
    return path


_lib = None


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_threads.argtypes = []
    L.oracle_threads.restype = i32
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_decode.restype = ctypes.c_double
    L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_e4m3_encode_array.argtypes = [p, i64, p]
    L.oracle_e4m3_encode_patterns.argtypes = [ctypes.c_uint32, i64, p]
    L.oracle_quantize_tiles.argtypes = [p, i64, i64, i64, i64, i64, p, i64, p, i64]
    L.oracle_quantize_tiles_mode.argtypes = [p, i64, i64, i64, i64, i64, i32, p, i64, p, i64]
    L.oracle_requant_1x128_to_128x1_mode.argtypes = [p, i64, i64, p, i32, p, p]
    L.oracle_dequantize_tiles.argtypes = [p, i64, i64, i64, i64, i64, p, i64, p, i64]
    L.oracle_requant_1x128_to_128x1.argtypes = [p, i64, i64, p, p, p]
    L.oracle_gemm_entries.argtypes = [p, i64, p, i64, p, i64, p, i64, i32, i64, p, p, i64, p, p]
    L.oracle_gemm.argtypes = [p, i64, p, i64, p, i64, p, i64, i32, i64, i64, i64, p, p]
    L.oracle_dgrad_entries.argtypes = [p, i64, p, i64, p, i64, p, i64, i64, p, p, i64, p, p]
    L.oracle_grouped_gemm_entries.argtypes = [p, i64, p, i64, p, i64, i64, p, i64, i64, p,
                                              i32, i64, p, p, i64, p, p]
    L.oracle_matmul_f32_entries.argtypes = [p, i64, p, i64, i64, p, p, i64, p, p]
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def use_library(path: str) -> None:
    """Route every call of this module to the oracle library at ``path`` (a
    build of the same source, e.g. ``build_native``)."""
    global _lib
    _lib = _bind(ctypes.CDLL(path))


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------- codec

def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: value of every code (NaN for 0x7F / 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y) -> np.ndarray:
    y = _c(np.atleast_1d(y), np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode_patterns(first: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint8)
    lib().oracle_e4m3_encode_patterns(first, count, _ptr(out))
    return out


# ---------------------------------------------------------------- quantizers

SCALE_FP32 = 0
SCALE_POW2 = 1


def quantize_tiles(x: np.ndarray, tile_rows: int, tile_cols: int, scale_mode: int = SCALE_FP32):
    """Quantize fp32 x[rows][cols] per tile_rows x tile_cols tile.

    scale_mode SCALE_FP32: s = fl32(amax/448); SCALE_POW2: s = the smallest
    power of two with 448*s >= amax (at least 2^-127).
    Returns (q uint8[rows][cols], s float32[ceil(rows/tr)][ceil(cols/tc)])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    nti, ntj = -(-rows // tile_rows), -(-cols // tile_cols)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((nti, ntj), np.float32)
    if scale_mode == SCALE_FP32:
        lib().oracle_quantize_tiles(_ptr(x), rows, cols, cols, tile_rows, tile_cols,
                                    _ptr(q), cols, _ptr(s), ntj)
    else:
        lib().oracle_quantize_tiles_mode(_ptr(x), rows, cols, cols, tile_rows, tile_cols,
                                         scale_mode, _ptr(q), cols, _ptr(s), ntj)
    return q, s


def quantize_act_1x128(x, scale_mode: int = SCALE_FP32):
    return quantize_tiles(x, 1, 128, scale_mode)


def quantize_act_128x1(x, scale_mode: int = SCALE_FP32):
    return quantize_tiles(x, 128, 1, scale_mode)


def quantize_weight_128x128(w, scale_mode: int = SCALE_FP32):
    return quantize_tiles(w, 128, 128, scale_mode)


def dequantize_tiles(q: np.ndarray, s: np.ndarray, tile_rows: int, tile_cols: int) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    rows, cols = q.shape
    v = np.empty((rows, cols), np.float32)
    lib().oracle_dequantize_tiles(_ptr(q), rows, cols, cols, tile_rows, tile_cols,
                                  _ptr(s), s.shape[1], _ptr(v), cols)
    return v


def requant_1x128_to_128x1(q: np.ndarray, s1: np.ndarray, scale_mode: int = SCALE_FP32):
    """Cached 1x128 codes q[rows][cols] + scales s1[rows][cols/128] ->
    128x1 codes q2[rows][cols] + scales s2[rows/128][cols] (same orientation)."""
    q = _c(q, np.uint8)
    s1 = _c(s1, np.float32)
    rows, cols = q.shape
    assert s1.shape == (rows, -(-cols // 128))
    q2 = np.empty((rows, cols), np.uint8)
    s2 = np.empty((-(-rows // 128), cols), np.float32)
    if scale_mode == SCALE_FP32:
        lib().oracle_requant_1x128_to_128x1(_ptr(q), rows, cols, _ptr(s1), _ptr(q2), _ptr(s2))
    else:
        lib().oracle_requant_1x128_to_128x1_mode(_ptr(q), rows, cols, _ptr(s1), scale_mode,
                                                 _ptr(q2), _ptr(s2))
    return q2, s2


# ---------------------------------------------------------------- GEMM

BSCALE_BLOCK128 = 0
BSCALE_ROW = 1


def gemm(qa, sa, qb, sb, bscale_mode: int = BSCALE_BLOCK128):
    """C = A B^T with per-128-K scales, in fp64; returns (C, T) float64[M][N].

    qa uint8[M][K], sa float32[M][K/128]; qb uint8[N][K];
    sb float32[N/128][K/128] (BLOCK128) or [N][K/128] (ROW)."""
    qa, qb = _c(qa, np.uint8), _c(qb, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    M, K = qa.shape
    N = qb.shape[0]
    assert K % 128 == 0 and qb.shape[1] == K
    c = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)
    lib().oracle_gemm(_ptr(qa), K, _ptr(sa), sa.shape[1], _ptr(qb), K, _ptr(sb), sb.shape[1],
                      bscale_mode, M, N, K, _ptr(c), _ptr(t))
    return c, t


def gemm_entries(qa, sa, qb, sb, idx_m, idx_n, bscale_mode: int = BSCALE_BLOCK128, K=None):
    """(C, T) at the given (m, n) pairs.  K defaults to the full width; a
    smaller multiple of 128 gives the prefix sum over the first K/128 chunks."""
    qa, qb = _c(qa, np.uint8), _c(qb, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    lda, ldb = qa.shape[1], qb.shape[1]
    K = lda if K is None else K
    assert K % 128 == 0 and K <= lda and K <= ldb
    im, jn = _c(idx_m, np.int64), _c(idx_n, np.int64)
    c = np.empty(im.size, np.float64)
    t = np.empty(im.size, np.float64)
    lib().oracle_gemm_entries(_ptr(qa), lda, _ptr(sa), sa.shape[1], _ptr(qb), ldb, _ptr(sb),
                              sb.shape[1], bscale_mode, K, _ptr(im), _ptr(jn), im.size,
                              _ptr(c), _ptr(t))
    return c, t


def matmul_f32_entries(x, w, idx_m, idx_n):
    """FP64 product of the unquantized inputs at selected outputs (reporting
    only): x float32[M][K], w float32[N][K]; returns (C, T) with
    C = sum_k x w and T = sum_k |x w| (float64 arrays)."""
    x, w = _c(x, np.float32), _c(w, np.float32)
    K = x.shape[1]
    assert w.shape[1] == K
    im, jn = _c(idx_m, np.int64), _c(idx_n, np.int64)
    c = np.empty(im.size, np.float64)
    t = np.empty(im.size, np.float64)
    lib().oracle_matmul_f32_entries(_ptr(x), K, _ptr(w), K, K, _ptr(im), _ptr(jn), im.size, _ptr(c), _ptr(t))
    return c, t


def grouped_gemm_entries(qa, sa, qb, sb, offsets, idx_m, idx_n):
    """Per-expert block-scaled GEMM at selected outputs.

    qa uint8[M][K], sa float32[M][K/128], qb uint8[G][N][K],
    sb float32[G][N/128][K/128], offsets int32[G+1]."""
    qa, qb = _c(qa, np.uint8), _c(qb, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    off = _c(offsets, np.int32)
    G, N, K = qb.shape
    im, jn = _c(idx_m, np.int64), _c(idx_n, np.int64)
    c = np.empty(im.size, np.float64)
    t = np.empty(im.size, np.float64)
    lib().oracle_grouped_gemm_entries(_ptr(qa), K, _ptr(sa), sa.shape[1], _ptr(qb), K, N * K,
                                      _ptr(sb), sb.shape[2], sb.shape[1] * sb.shape[2],
                                      _ptr(off), G, K, _ptr(im), _ptr(jn), im.size,
                                      _ptr(c), _ptr(t))
    return c, t


def dgrad_entries(qdy, sdy, qw, sw, idx_m, idx_k):
    """dX = dY W at selected (m, k): qdy uint8[M][N] with 1x128 scales
    sdy float32[M][N/128]; qw uint8[N][K] with block scales
    sw float32[N/128][ceil(K/128)].  Returns (C, T) float64 arrays."""
    qdy, qw = _c(qdy, np.uint8), _c(qw, np.uint8)
    sdy, sw = _c(sdy, np.float32), _c(sw, np.float32)
    M, N = qdy.shape
    assert N % 128 == 0 and qw.shape[0] == N
    im, ik = _c(idx_m, np.int64), _c(idx_k, np.int64)
    c = np.empty(im.size, np.float64)
    t = np.empty(im.size, np.float64)
    lib().oracle_dgrad_entries(_ptr(qdy), N, _ptr(sdy), sdy.shape[1], _ptr(qw), qw.shape[1], _ptr(sw),
                               sw.shape[1], N, _ptr(im), _ptr(ik), im.size, _ptr(c), _ptr(t))
    return c, t


def dgrad(qdy, sdy, qw, sw):
    """Every output of dgrad_entries: (C, T) float64[M][K]."""
    M = qdy.shape[0]
    K = qw.shape[1]
    mm, kk = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    c, t = dgrad_entries(qdy, sdy, qw, sw, mm.ravel(), kk.ravel())
    return c.reshape(M, K), t.reshape(M, K)


def gather_quantize_act_1x128(x: np.ndarray, row_index: np.ndarray, scale_mode: int = SCALE_FP32):
    """MoE dispatch in FP8 (page 2, xn--jj0bz6z98ct0a29q.com wr_id=362465, and
    page 3, why-be.why-be.co.kr wr_id=55081, passages on dispatching
    activations in FP8): output row i is row row_index[i] of x, quantized per
    1x128 tile; an index outside [0, rows) stands for an empty slot and gives
    a zero row (scale 0, codes 0x00).  The gather is a plain row selection;
    the quantization is quantize_act_1x128.
    Returns (q uint8[len(idx)][cols], s float32[len(idx)][ceil(cols/128)])."""
    x = _c(x, np.float32)
    idx = np.asarray(row_index, dtype=np.int64)
    valid = (idx >= 0) & (idx < x.shape[0])
    g = np.zeros((idx.size, x.shape[1]), np.float32)
    g[valid] = x[idx[valid]]
    return quantize_tiles(g, 1, 128, scale_mode)
