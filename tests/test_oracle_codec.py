"""Pins of the oracle's E4M3FN codec against the format definition.

The oracle's decode table and encoder are compared with values derived by
hand (tests/golden/e4m3_hand_values.txt), with an exact rational model of the
format (tests/exact.py), and exhaustively over every non-negative finite fp32
bit pattern against an independent threshold construction.
"""
import os

import numpy as np
import pytest

from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_values():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_hand_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, code = line.split()[:2]
            out.append((float(v), int(code, 16)))
    return out


def test_decode_table_matches_format(oracle):
    table = oracle.e4m3_decode_table()
    for code in range(256):
        if code & 0x7F == 0x7F:
            assert np.isnan(table[code])
        else:
            assert table[code] == float(exact.e4m3_value(code)), hex(code)
    # spot values of the format
    assert table[0x38] == 1.0 and table[0x7E] == 448.0 and table[0x08] == 2.0 ** -6
    assert table[0x01] == 2.0 ** -9 and table[0x80] == 0.0 and np.signbit(table[0x80])
    finite = table[np.isfinite(table)]
    assert finite.size == 254 and np.max(np.abs(finite)) == 448.0


def test_hand_values(oracle):
    for v, code in _hand_values():
        assert oracle.e4m3_encode(np.float32(v))[0] == code, (v, hex(code))


def test_encode_matches_bruteforce_sample(oracle):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x43E80000, size=4000, dtype=np.uint32)  # |y| < 464
    bits[::2] |= np.uint32(0x80000000)
    ys = bits.view(np.float32)
    got = oracle.e4m3_encode(ys)
    for y, g in zip(ys, got):
        assert g == exact.e4m3_nearest(float(y)), (float(y), hex(g))


def _boundaries():
    """fp32 bit patterns of the midpoints between consecutive magnitudes."""
    mags = [float(v) for _, v in exact.e4m3_magnitudes()]
    mids = [(mags[i] + mags[i + 1]) / 2 for i in range(126)]
    b = np.array(mids, dtype=np.float32).view(np.uint32)
    # every midpoint is exactly representable in fp32
    assert np.all(b.view(np.float32).astype(np.float64) == np.array(mids))
    return b


def _expected_codes(first: int, count: int, bounds: np.ndarray) -> np.ndarray:
    """Expected code of each non-negative pattern in [first, first+count): the
    number of midpoints strictly below it, and at a midpoint the even of the two
    neighbouring codes.  Built as a step function over the (sorted) range."""
    last = first + count
    codes = np.empty(count, np.uint8)
    # code c covers patterns (bounds[c-1], bounds[c]) exclusive of ties
    lo_idx = int(np.searchsorted(bounds, np.uint32(first), side="left"))
    pos = first
    c = lo_idx
    while pos < last:
        nxt = int(bounds[c]) if c < bounds.size else last  # first pattern of the tie at the next midpoint
        seg_end = min(nxt, last)
        codes[pos - first:seg_end - first] = c
        pos = seg_end
        if pos < last and c < bounds.size and pos == int(bounds[c]):
            codes[pos - first] = c if c % 2 == 0 else c + 1  # tie at the midpoint
            pos += 1
        c += 1
    return codes


SAT_START = 0x43E80000  # 464.0: every larger finite magnitude saturates


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_encode_exhaustive(oracle, sign):
    """All fp32 patterns with |y| < 464 of one sign, then a strided sample of
    the saturating range up to the largest finite value."""
    bounds = _boundaries()
    chunk = 1 << 26
    for first in range(0, SAT_START, chunk):
        count = min(chunk, SAT_START - first)
        got = oracle.e4m3_encode_patterns(sign + first, count)
        exp = _expected_codes(first, count, bounds) | np.uint8(0x80 if sign else 0)
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, f"pattern {sign + first + int(bad[0]):#010x}: {got[bad[0]]:#x} vs {exp[bad[0]]:#x}"
    pats = np.arange(SAT_START, 0x7F800000, 4099, dtype=np.uint64).astype(np.uint32) | np.uint32(sign)
    got = oracle.e4m3_encode(pats.view(np.float32))
    assert np.all(got == np.uint8(0x7E | (0x80 if sign else 0)))


def test_roundtrip_of_every_code(oracle):
    table = oracle.e4m3_decode_table()
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(np.float32(table[code]))[0] == code
