"""Pins of the oracle's power-of-two scale variant (scale_mode SCALE_POW2).

Rule: s = the smallest power of two with 448 * s >= amax (at least 2^-127,
0 for an all-zero tile), q = e4m3(fl32(x / s)).  Pinned against a hand
derivation (tests/golden/pow2_scale_tile_codes.txt), a closed form of the
scale evaluated with exact rationals (tests/exact.py), invariants checked on
the fp32 bit patterns, agreement with the fp32-scale rule where the two
coincide, special cases, and lossless requantization.
"""
import os
import zlib

import numpy as np
import pytest

from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
POW2 = 1


def _golden():
    out = []
    with open(os.path.join(GOLDEN, "pow2_scale_tile_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                j, c = line.split()
                out.append((int(j), int(c, 16)))
    return out


@pytest.mark.parametrize("p", [0, -7, 5, 60, -60, -119])
def test_power_of_two_tile(oracle, p):
    codes = _golden()
    x = np.zeros((1, 128), np.float32)
    for j, _ in codes:
        x[0, j] = np.float32(2.0 ** (p - j))
    q, s = oracle.quantize_act_1x128(x, POW2)
    assert s[0, 0] == np.float32(2.0 ** (p - 8))
    for j, c in codes:
        assert q[0, j] == c, (p, j, hex(q[0, j]), hex(c))
    v = oracle.dequantize_tiles(q, s, 1, 128)
    for j, _ in codes:
        if j <= 17:
            assert v[0, j] == x[0, j]


def _matrix(rng, rows, cols, kind):
    if kind == "normal":
        return rng.standard_normal((rows, cols)).astype(np.float32)
    if kind == "bf16":
        a = rng.standard_t(3, (rows, cols)).astype(np.float32)
        return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    if kind == "wide":
        e = rng.integers(-140, 30, size=(rows, cols))
        return (rng.choice([-1.0, 1.0], (rows, cols)) * rng.random((rows, cols)) * np.exp2(e)).astype(np.float32)
    if kind == "tiny":
        return (rng.standard_normal((rows, cols)) * 1e-38).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("tile", [(1, 128), (128, 1), (128, 128), (2, 40)])
@pytest.mark.parametrize("kind", ["normal", "bf16", "wide", "tiny"])
def test_matches_exact_rule(oracle, tile, kind):
    rng = np.random.default_rng(zlib.crc32(repr(("pow2", tile, kind)).encode()))
    tr, tc = tile
    rows, cols = (3, 300) if tr == 1 else (150, 3) if tc == 1 else (130, 131) if tr == 128 else (5, 90)
    x = _matrix(rng, rows, cols, kind)
    x[0, 0] = -0.0
    q, s = oracle.quantize_tiles(x, tr, tc, POW2)
    for I in range(-(-rows // tr)):
        for J in range(-(-cols // tc)):
            sl = (slice(I * tr, min(rows, I * tr + tr)), slice(J * tc, min(cols, J * tc + tc)))
            codes, sc = exact.quantize_tile_exact_pow2(float(v) for v in x[sl].ravel())
            assert s[I, J] == np.float32(sc), (I, J, s[I, J], sc)
            assert list(q[sl].ravel()) == codes, (I, J)


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny"])
def test_scale_invariants(oracle, kind):
    """Checked on the stored bits: s is a power of two (one bit set in a
    normal or subnormal fp32), 448 s >= amax, and either s = 2^-127 or the
    next smaller power of two would be too small (224 s < amax)."""
    rng = np.random.default_rng(7)
    x = _matrix(rng, 64, 1024, kind)
    _, s = oracle.quantize_act_1x128(x, POW2)
    amax = np.abs(x).reshape(64, 8, 128).max(axis=2).astype(np.float64)
    sd = s.astype(np.float64)
    bits = s.view(np.uint32)
    expo, mant = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    one_bit = (mant == 0) | ((expo == 0) & ((mant & (mant - 1)) == 0))
    assert np.all(one_bit[amax > 0])
    assert np.all(448.0 * sd >= amax)
    assert np.all((sd == 2.0 ** -127) | (224.0 * sd < amax))
    assert np.all(s[amax == 0] == 0)


def test_agrees_with_fp32_rule_when_amax_is_448_times_power_of_two(oracle):
    """amax = 448 * 2^k gives s = 2^k under both rules, hence equal codes."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 1024)).astype(np.float32)
    k = rng.integers(-30, 30, size=(32, 8))
    for r in range(32):
        for j in range(8):
            blk = x[r, 128 * j:128 * j + 128]
            blk *= np.float32(448.0 * 2.0 ** k[r, j]) / np.abs(blk).max()
            blk[np.argmax(np.abs(blk))] = np.float32(448.0 * 2.0 ** k[r, j])
    q0, s0 = oracle.quantize_act_1x128(x)
    q1, s1 = oracle.quantize_act_1x128(x, POW2)
    assert np.array_equal(s0, s1) and np.array_equal(s1, np.exp2(k).astype(np.float32))
    assert np.array_equal(q0, q1)


def test_special_cases(oracle):
    x = np.zeros((4, 128), np.float32)
    x[1, 5] = -0.0
    x[2, :] = np.float32(2.0 ** -140)       # needs 2^-148: clamped to 2^-127
    x[3, 0] = np.float32(3.4e38)            # largest scales: 2^120
    q, s = oracle.quantize_act_1x128(x, POW2)
    assert s[0, 0] == 0 and s[1, 0] == 0 and np.all(q[0] == 0)
    assert q[1, 5] == 0x80
    assert s[2, 0] == np.float32(2.0 ** -127)
    assert np.all(q[2] == exact.e4m3_nearest(float(np.float32(2.0 ** -13))))  # 2^-140 / 2^-127
    assert s[3, 0] == np.float32(2.0 ** 120)


@pytest.mark.parametrize("tile", [(1, 128), (128, 1), (128, 128)])
def test_roundtrip_bound(oracle, tile):
    """|x - s dec(q)| <= max(2^-4 |x|, 2^-10 s): half a normal E4M3 spacing,
    or half the subnormal spacing in scaled units."""
    rng = np.random.default_rng(4)
    x = (rng.standard_t(3, (256, 384)) * np.exp2(rng.integers(-20, 20, (256, 1)))).astype(np.float32)
    q, s = oracle.quantize_tiles(x, *tile, POW2)
    v = oracle.dequantize_tiles(q, s, *tile).astype(np.float64)
    srep = np.repeat(np.repeat(s.astype(np.float64), tile[0], 0)[:256], tile[1], 1)[:, :384]
    err = np.abs(x.astype(np.float64) - v)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * srep))


def test_requant_is_lossless_for_normal_codes(oracle):
    """With power-of-two scales, dec(q) * s1 is exact and the 128x1 scale s2
    differs from s1 by a power of two; codes of magnitude >= 2 with s1 within
    2^3 of each other stay normal after rescaling, so requantization keeps
    every value: dequant(q2, s2) == dequant(q, s1) bit for bit."""
    rng = np.random.default_rng(5)
    rows, cols = 256, 384
    e = rng.integers(8, 16, (rows, cols))                   # exponent fields: values >= 2
    m = rng.integers(0, 8, (rows, cols))
    m[e == 15] = rng.integers(0, 7, int((e == 15).sum()))   # avoid NaN codes
    q = ((rng.integers(0, 2, (rows, cols)) << 7) | (e << 3) | m).astype(np.uint8)
    s1 = np.exp2(rng.integers(-3, 4, (rows, cols // 128))).astype(np.float32)
    q2, s2 = oracle.requant_1x128_to_128x1(q, s1, POW2)
    v1 = oracle.dequantize_tiles(q, s1, 1, 128)
    v2 = oracle.dequantize_tiles(q2, s2, 128, 1)
    assert np.array_equal(v1, v2)


def test_requant_is_dequant_then_pow2_quantize(oracle):
    rng = np.random.default_rng(6)
    x = rng.standard_t(3, (300, 260)).astype(np.float32)
    q, s1 = oracle.quantize_act_1x128(x, POW2)
    v = oracle.dequantize_tiles(q, s1, 1, 128)
    qe, se = oracle.quantize_act_128x1(v, POW2)
    q2, s2 = oracle.requant_1x128_to_128x1(q, s1, POW2)
    assert np.array_equal(q2, qe) and np.array_equal(s2, se)
