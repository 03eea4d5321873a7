"""The C-ABI library loads, exports every symbol of include/fp8q.h, and
rejects invalid arguments on the host before anything is launched (these
calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp8q_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def lib():
    import fp8_fine_grained_x128_amd as f
    return f


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_requant_transpose", "fp8q_gemm",
              "fp8q_grouped_gemm", "fp8q_strerror"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(fp8q_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in _declared():
        assert getattr(raw, n) is not None


def test_strerror_and_version(lib):
    assert lib.fp8q_strerror(0) == "ok"
    for s in range(1, 6):
        assert lib.fp8q_strerror(s) and lib.fp8q_strerror(s) != "ok"
    assert lib.fp8q_strerror(99) == "unknown status"
    assert lib.fp8q_version() >= 100


FAKE = 1 << 20  # an aligned, never-dereferenced address


def test_quantize_act_validation(lib):
    q = lib.fp8q_quantize_act
    assert q(FAKE, 7, 4, 128, 128, 0, FAKE, 128, FAKE, 4) == lib.FP8Q_EINVAL  # dtype
    assert q(FAKE, 1, 4, 128, 128, 5, FAKE, 128, FAKE, 4) == lib.FP8Q_EINVAL  # tile
    assert q(FAKE, 1, -1, 128, 128, 0, FAKE, 128, FAKE, 4) == lib.FP8Q_ESHAPE
    assert q(FAKE, 1, 4, 128, 64, 0, FAKE, 128, FAKE, 4) == lib.FP8Q_ESHAPE  # ldx < cols
    assert q(FAKE, 1, 4, 128, 128, 0, FAKE, 128, FAKE, 3) == lib.FP8Q_ESHAPE  # lds < rows
    assert q(FAKE, 1, 4, 128, 128, 1, FAKE, 3, FAKE, 128) == lib.FP8Q_ESHAPE  # 128x1: ldq < rows
    assert q(0, 1, 4, 128, 128, 0, FAKE, 128, FAKE, 4) == lib.FP8Q_EINVAL  # null
    assert q(FAKE + 2, 1, 4, 128, 128, 0, FAKE, 128, FAKE, 4) == lib.FP8Q_EALIGN
    assert q(FAKE, 1, 4, 100, 100, 0, FAKE, 112, FAKE, 4) == lib.FP8Q_EALIGN  # ldx*2 % 16
    assert q(FAKE, 1, 4, 128, 128, 0, FAKE, 130, FAKE, 4) == lib.FP8Q_EALIGN  # ldq % 16
    assert q(0, 1, 0, 128, 128, 0, 0, 128, 0, 0) == lib.FP8Q_OK  # empty: nothing launched


def test_quantize_weight_and_requant_validation(lib):
    w = lib.fp8q_quantize_weight
    assert w(FAKE, 0, 256, 512, 512, FAKE, 512, FAKE, 3) == lib.FP8Q_ESHAPE  # lds < K/128
    assert w(FAKE, 2, 256, 512, 512, FAKE, 512, FAKE, 4) == lib.FP8Q_EINVAL
    assert w(FAKE, 0, 256, 512, 512, 0, 512, FAKE, 4) == lib.FP8Q_EINVAL
    assert w(FAKE, 0, 0, 512, 512, 0, 512, 0, 4) == lib.FP8Q_OK
    r = lib.fp8q_requant_transpose
    assert r(FAKE, 256, 256, 256, FAKE, 256, FAKE, 255, FAKE, 256) == lib.FP8Q_ESHAPE
    assert r(FAKE, 256, 256, 256, FAKE, 256, FAKE, 256, 0, 256) == lib.FP8Q_EINVAL
    assert r(FAKE + 8, 256, 256, 256, FAKE, 256, FAKE, 256, FAKE, 256) == lib.FP8Q_EALIGN


def test_gemm_validation(lib):
    g = lib.fp8q_gemm
    ok = dict(a=FAKE, lda=256, sa=FAKE, ldsa=64, b=FAKE, ldb=256, sb=FAKE, ldsb=2, bscale=0, M=64,
              N=64, K=256, c=FAKE, c_dtype=0, ldc=64, accumulate=0)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return g(*d.values())

    assert call(K=200) == lib.FP8Q_ESHAPE
    assert call(K=0) == lib.FP8Q_ESHAPE
    assert call(lda=128) == lib.FP8Q_ESHAPE
    assert call(ldsa=63) == lib.FP8Q_ESHAPE
    assert call(ldsb=1) == lib.FP8Q_ESHAPE
    assert call(bscale=1, ldsb=63) == lib.FP8Q_ESHAPE
    assert call(bscale=2) == lib.FP8Q_EINVAL
    assert call(c_dtype=3) == lib.FP8Q_EINVAL
    assert call(a=0) == lib.FP8Q_EINVAL
    assert call(a=FAKE + 4) == lib.FP8Q_EALIGN
    assert call(lda=264) == lib.FP8Q_EALIGN
    assert call(c_dtype=1, accumulate=1) == lib.FP8Q_EUNSUPPORTED
    assert call(M=0, a=0, b=0, c=0) == lib.FP8Q_OK


def test_grouped_validation(lib):
    g = lib.fp8q_grouped_gemm
    ok = dict(a=FAKE, lda=256, sa=FAKE, ldsa=64, b=FAKE, ldb=256, bgs=256 * 128, sb=FAKE, ldsb=2,
              sbgs=2, off=FAKE, G=4, M=64, N=128, K=256, c=FAKE, c_dtype=1, ldc=128)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return g(*d.values())

    assert call(G=0) == lib.FP8Q_ESHAPE
    assert call(G=5000) == lib.FP8Q_ESHAPE
    assert call(off=0) == lib.FP8Q_EINVAL
    assert call(bgs=100) == lib.FP8Q_ESHAPE
    assert call(sbgs=1) == lib.FP8Q_ESHAPE
    assert call(off=FAKE + 2) == lib.FP8Q_EALIGN


def test_gemm_ex_flags(lib):
    ok = [FAKE, 256, FAKE, 64, FAKE, 256, FAKE, 2, 0, 64, 64, 256, FAKE, 0, 64, 0]
    assert lib.fp8q_gemm_ex(*ok, 1 << 7) == lib.FP8Q_EINVAL  # unknown flag bit
    assert lib.fp8q_gemm_ex(*ok[:11], 200, *ok[12:], lib.FP8Q_GEMM_MMA_FP8) == lib.FP8Q_ESHAPE
    g = [FAKE, 256, FAKE, 64, FAKE, 256, 256 * 128, FAKE, 2, 2, FAKE, 4, 64, 128, 256, FAKE, 1, 128]
    assert lib.fp8q_grouped_gemm_ex(*g, 1 << 9) == lib.FP8Q_EINVAL
    assert lib.fp8q_grouped_gemm_ex(*g[:11], 0, *g[12:], lib.FP8Q_GEMM_MMA_FP8) == lib.FP8Q_ESHAPE


def test_quantize_ex_scale_mode(lib):
    assert lib.fp8q_quantize_act_ex(FAKE, 1, 4, 128, 128, 0, FAKE, 128, FAKE, 4, 2) == lib.FP8Q_EINVAL
    assert lib.fp8q_quantize_act_ex(FAKE, 1, 4, 128, 64, 0, FAKE, 128, FAKE, 4, 1) == lib.FP8Q_ESHAPE
    assert lib.fp8q_quantize_weight_ex(FAKE, 0, 256, 512, 512, FAKE, 512, FAKE, 4, -1) == lib.FP8Q_EINVAL
    assert lib.fp8q_quantize_weight_ex(FAKE, 0, 0, 512, 512, 0, 512, 0, 4, 1) == lib.FP8Q_OK
    assert lib.fp8q_requant_transpose_ex(FAKE, 256, 256, 256, FAKE, 256, FAKE, 256, FAKE, 256, 3) == \
        lib.FP8Q_EINVAL
    assert lib.fp8q_requant_transpose_ex(FAKE, 256, 256, 256, FAKE, 256, FAKE, 255, FAKE, 256, 1) == \
        lib.FP8Q_ESHAPE


def test_transpose_weight_validation(lib):
    t = lib.fp8q_transpose_weight
    assert t(FAKE, 256, 384, 383, FAKE, 3, FAKE, 256, FAKE, 2) == lib.FP8Q_ESHAPE  # ldq < K
    assert t(FAKE, 256, 384, 384, FAKE, 2, FAKE, 256, FAKE, 2) == lib.FP8Q_ESHAPE  # lds < K/128
    assert t(FAKE, 256, 384, 384, FAKE, 3, FAKE, 255, FAKE, 2) == lib.FP8Q_ESHAPE  # ldqt < N
    assert t(FAKE, 256, 384, 384, FAKE, 3, FAKE, 256, FAKE, 1) == lib.FP8Q_ESHAPE  # ldst < N/128
    assert t(0, 256, 384, 384, FAKE, 3, FAKE, 256, FAKE, 2) == lib.FP8Q_EINVAL
    assert t(FAKE + 8, 256, 384, 384, FAKE, 3, FAKE, 256, FAKE, 2) == lib.FP8Q_EALIGN
    assert t(0, 0, 384, 384, 0, 3, 0, 0, 0, 0) == lib.FP8Q_OK


def test_gather_quantize_validation(lib):
    g = lib.fp8q_gather_quantize_act
    assert g(FAKE, 1, 10, 128, 128, FAKE, 4, FAKE, 128, FAKE, 4, 2) == lib.FP8Q_EINVAL  # scale mode
    assert g(FAKE, 5, 10, 128, 128, FAKE, 4, FAKE, 128, FAKE, 4, 0) == lib.FP8Q_EINVAL  # dtype
    assert g(FAKE, 1, 10, 128, 128, 0, 4, FAKE, 128, FAKE, 4, 0) == lib.FP8Q_EINVAL    # index
    assert g(FAKE, 1, 10, 128, 127, FAKE, 4, FAKE, 128, FAKE, 4, 0) == lib.FP8Q_ESHAPE  # ldx
    assert g(FAKE, 1, 10, 128, 128, FAKE, 4, FAKE, 128, FAKE, 3, 0) == lib.FP8Q_ESHAPE  # lds < rows_out
    assert g(FAKE, 1, 10, 128, 128, FAKE + 2, 4, FAKE, 128, FAKE, 4, 0) == lib.FP8Q_EALIGN
    assert g(0, 1, 10, 128, 128, 0, 0, 0, 128, 0, 0, 0) == lib.FP8Q_OK  # no rows out


def test_gemm_rejects_huge_row_strides(lib):
    big = 1 << 24
    assert lib.fp8q_gemm(FAKE, big, FAKE, 64, FAKE, 256, FAKE, 2, 0, 64, 64, 256, FAKE, 0, 64, 0) == \
        lib.FP8Q_EUNSUPPORTED
    assert lib.fp8q_gemm(FAKE, 256, FAKE, 64, FAKE, big, FAKE, 2, 0, 64, 64, 256, FAKE, 0, 64, 0) == \
        lib.FP8Q_EUNSUPPORTED


def test_splitk_plan_and_validation(lib):
    """Split-K: the workspace query follows the documented plan (slices =
    compute units / 256x256 tiles, at least 4 chunks each, only when the tiles
    fill at most half the GPU), and the workspace is validated on the host.
    Without a GPU the library plans for 256 compute units."""
    ws = lib.fp8q_gemm_splitk_workspace
    assert ws(4096, 7168, 7168) == 0          # 448 tiles: no split
    assert ws(1024, 1024, 65536) == 16 * 1024 * 1024 * 4  # 16 tiles x 16 slices of 32 chunks
    assert ws(1000, 1000, 65536) == 16 * 1000 * 1000 * 4  # ldws = N rounded up to 4
    assert ws(1024, 1023, 65536) == 16 * 1024 * 1024 * 4
    assert ws(256, 256, 1024) == 2 * 256 * 256 * 4        # 8 chunks: 2 slices of 4
    assert ws(256, 256, 512) == 0                         # 4 chunks: too short to split
    assert ws(1024, 1024, 100) == 0 and ws(0, 1024, 65536) == 0 and ws(1024, 1024, -128) == 0
    g = lib.fp8q_gemm_splitk
    need = ws(1024, 1024, 65536)
    args = (FAKE, 65536, FAKE, 1024, FAKE, 65536, FAKE, 512, 0, 1024, 1024, 65536, FAKE, 0, 1024, 0, 0)
    assert g(*args, 0, need) == lib.FP8Q_EINVAL               # no workspace where one is needed
    assert g(*args, FAKE, need - 4) == lib.FP8Q_ESHAPE        # too small
    assert g(*args, FAKE + 16, need) == lib.FP8Q_EALIGN       # not 256-byte aligned
    assert g(*args, FAKE, -1) == lib.FP8Q_ESHAPE
    bad_k = args[:11] + (65536 + 64,) + args[12:]
    assert g(*bad_k, FAKE, need) == lib.FP8Q_ESHAPE           # K % 128
    assert g(*args[:16], 4, FAKE, need) == lib.FP8Q_EINVAL    # unknown flag


def test_clock_probe_validation(lib):
    p = lib.fp8q_clock_probe
    assert p(0, 1000) == lib.FP8Q_EINVAL
    assert p(FAKE + 4, 1000) == lib.FP8Q_EALIGN
    assert p(FAKE, 0) == lib.FP8Q_ESHAPE
    assert p(FAKE, 100000001) == lib.FP8Q_ESHAPE
