"""Pins of the oracle's tile quantizers and 1x128 -> 128x1 requantization.

Pinned against: closed forms (power-of-two tiles, exact tiles), an exact
rational evaluation of the quantization rule on random tiles of every shape
(tests/exact.py), the round-trip error bound of the format, and special cases
(zero tiles, signed zeros, subnormal scales, partial tiles).
"""
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest

from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pow2_codes():
    out = []
    with open(os.path.join(GOLDEN, "pow2_tile_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                j, c = line.split()
                out.append((int(j), int(c, 16)))
    return out


@pytest.mark.parametrize("p", [0, -7, 5, 60, -60])
def test_power_of_two_tile(oracle, p):
    codes = _pow2_codes()
    x = np.zeros((1, 128), np.float32)
    for j, _ in codes:
        x[0, j] = np.float32(2.0 ** (p - j))
    q, s = oracle.quantize_act_1x128(x)
    assert s[0, 0] == np.float32(2.0 ** p) / np.float32(448.0)
    for j, c in codes:
        assert q[0, j] == c, (p, j, hex(q[0, j]), hex(c))
    assert np.all(q[0, len(codes):] == 0)
    v = oracle.dequantize_tiles(q, s, 1, 128)
    for j, _ in codes:
        if j <= 15:
            assert v[0, j] == x[0, j]


@pytest.mark.parametrize("p", [0, -20, 9])
def test_exact_tiles_roundtrip(oracle, p):
    """amax = 448 * 2^p gives s = 2^p exactly; entries +-2^(p+i), i in [-9, 8],
    are E4M3 values times s and come back bit-exactly."""
    rng = np.random.default_rng(3)
    i = rng.integers(-9, 9, size=(256, 256))
    sign = rng.choice([-1.0, 1.0], size=(256, 256))
    x = (sign * np.exp2(p + i)).astype(np.float32)
    x[::128, ::128] = np.float32(448.0 * 2.0 ** p)  # one amax per 128x128 block, 1x128 tile
    x[:, ::128] = np.float32(448.0 * 2.0 ** p)
    for tr, tc in [(1, 128), (128, 1), (128, 128)]:
        q, s = oracle.quantize_tiles(x, tr, tc)
        if (tr, tc) == (128, 1):
            continue  # 128x1 tiles of this matrix do not all contain an amax entry
        assert np.all(s == np.float32(2.0 ** p))
        v = oracle.dequantize_tiles(q, s, tr, tc)
        assert np.array_equal(v, x)


def _random_tile_matrix(rng, rows, cols, kind):
    if kind == "normal":
        return rng.standard_normal((rows, cols)).astype(np.float32)
    if kind == "bf16":
        a = rng.standard_t(3, (rows, cols)).astype(np.float32)
        return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # bf16-representable
    if kind == "wide":
        e = rng.integers(-140, 30, size=(rows, cols))
        return (rng.choice([-1.0, 1.0], (rows, cols)) * rng.random((rows, cols)) * np.exp2(e)).astype(np.float32)
    if kind == "tiny":  # subnormal-range scales
        return (rng.standard_normal((rows, cols)) * 1e-38).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("tile", [(1, 128), (128, 1), (128, 128), (2, 40)])
@pytest.mark.parametrize("kind", ["normal", "bf16", "wide", "tiny"])
def test_quantize_matches_exact_rule(oracle, tile, kind):
    """Every code and scale equals the exact-rational evaluation of
    s = fl32(amax/448), q = e4m3(fl32(x/s)) on a ragged matrix."""
    rng = np.random.default_rng(zlib.crc32(repr((tile, kind)).encode()))
    tr, tc = tile
    rows, cols = (3, 300) if tr == 1 else (150, 3) if tc == 1 else (130, 131) if tr == 128 else (5, 90)
    x = _random_tile_matrix(rng, rows, cols, kind)
    x[0, 0] = -0.0
    q, s = oracle.quantize_tiles(x, tr, tc)
    for I in range(-(-rows // tr)):
        for J in range(-(-cols // tc)):
            sl = (slice(I * tr, min(rows, I * tr + tr)), slice(J * tc, min(cols, J * tc + tc)))
            vals = [float(v) for v in x[sl].ravel()]
            codes, sc = exact.quantize_tile_exact(vals)
            assert s[I, J] == np.float32(sc), (I, J)
            assert list(q[sl].ravel()) == codes, (I, J)


def test_zero_and_signed_zero_tiles(oracle):
    x = np.zeros((2, 256), np.float32)
    x[0, 5] = -0.0
    x[1, 128:] = -0.0
    q, s = oracle.quantize_act_1x128(x)
    assert np.all(s == 0)
    assert q[0, 5] == 0x80 and q[0, 4] == 0x00
    assert np.all(q[1, 128:] == 0x80) and np.all(q[1, :128] == 0)


def test_scale_underflow_gives_signed_zeros(oracle):
    tiny = np.float32(1.4e-45)  # smallest subnormal: amax/448 rounds to 0
    x = np.array([[tiny, -tiny] + [0.0] * 126], np.float32)
    q, s = oracle.quantize_act_1x128(x)
    assert s[0, 0] == 0 and q[0, 0] == 0x00 and q[0, 1] == 0x80


def test_partial_tiles_use_valid_elements_only(oracle):
    x = np.ones((1, 130), np.float32)
    x[0, 129] = 8.0  # second (partial) tile has 2 valid elements
    q, s = oracle.quantize_act_1x128(x)
    assert s[0, 0] == np.float32(1.0) / np.float32(448.0)
    assert s[0, 1] == np.float32(8.0) / np.float32(448.0)
    assert q.shape == (1, 130) and s.shape == (1, 2)


@pytest.mark.parametrize("tile", [(1, 128), (128, 1), (128, 128)])
def test_roundtrip_bound(oracle, tile):
    """|x - s*dec(q)| <= max(2^-4 |x|, 2^-10 s): half a unit in the last place
    of E4M3 in the normal range (3 mantissa bits), half the subnormal spacing
    2^-9 below it."""
    rng = np.random.default_rng(11)
    x = rng.standard_t(3, (256, 384)).astype(np.float32)
    x[:, 7] *= 100
    q, s = oracle.quantize_tiles(x, *tile)
    d = oracle.e4m3_decode_table()[q].astype(np.float64)
    s_full = np.repeat(np.repeat(s, tile[0], axis=0), tile[1], axis=1)[: x.shape[0], : x.shape[1]].astype(np.float64)
    err = np.abs(x.astype(np.float64) - s_full * d)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s_full) * (1 + 1e-6)
    assert np.all(err <= bound)
    # in every tile the largest magnitude maps onto 448 (or the code just below)
    R, C = x.shape
    tmax = np.abs(d).reshape(R // tile[0], tile[0], C // tile[1], tile[1]).max(axis=(1, 3))
    assert np.all(tmax >= 416)


def test_requant_is_dequant_then_128x1(oracle):
    """requant = quantize_128x1(fl32(dec(q) * s)) with the exact rule."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256 + 17, 256 + 40)).astype(np.float32)
    q1, s1 = oracle.quantize_act_1x128(x)
    q2, s2 = oracle.requant_1x128_to_128x1(q1, s1)
    v = oracle.dequantize_tiles(q1, s1, 1, 128)
    # dequantized values are fp32 products of the code value and the scale
    for r, c in [(0, 0), (100, 200), (272, 295)]:
        assert v[r, c] == exact.round_f32(exact.e4m3_value(int(q1[r, c])) * Fraction(float(s1[r, c // 128])))
    for J in [0, 5, 295]:
        for I in range(3):
            rows = slice(128 * I, min(v.shape[0], 128 * I + 128))
            codes, sc = exact.quantize_tile_exact([float(t) for t in v[rows, J]])
            assert s2[I, J] == np.float32(sc)
            assert list(q2[rows, J]) == codes


def test_requant_of_exact_powers_is_lossless(oracle):
    """Power-of-two data whose 128x1 tiles hold +-448*2^p: requantization
    reproduces the same values exactly."""
    rng = np.random.default_rng(8)
    x = np.exp2(rng.integers(-6, 8, size=(256, 256))).astype(np.float32)
    x[0, :] = 448.0
    x[128, :] = 448.0
    x[:, 0] = 448.0
    q1, s1 = oracle.quantize_act_1x128(x)
    assert np.array_equal(oracle.dequantize_tiles(q1, s1, 1, 128), x)
    q2, s2 = oracle.requant_1x128_to_128x1(q1, s1)
    assert np.array_equal(oracle.dequantize_tiles(q2, s2, 128, 1), x)


def test_gather_quantize_is_row_selection_then_quantize(oracle):
    """Each output row equals the 1x128 quantization of its source row alone
    (rows are independent under 1x128 tiles), repeated sources give equal
    rows, and empty slots (-1, out of range) give zero codes and scale 0."""
    rng = np.random.default_rng(21)
    x = rng.standard_t(3, (40, 300)).astype(np.float32)
    idx = np.array([5, 5, 39, 0, -1, 40, 17, 5], np.int64)
    q, s = oracle.gather_quantize_act_1x128(x, idx)
    for i, r in enumerate(idx):
        if 0 <= r < 40:
            qr, sr = oracle.quantize_act_1x128(x[r:r + 1])
            assert np.array_equal(q[i], qr[0]) and np.array_equal(s[i], sr[0])
        else:
            assert np.all(q[i] == 0) and np.all(s[i] == 0)
    assert np.array_equal(q[0], q[1]) and np.array_equal(q[0], q[7])
