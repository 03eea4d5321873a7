"""Pins of the oracle's block-scaled GEMM (plain, Wgrad row-scaled, grouped).

Pinned against: exact rational brute force on small shapes (every chunk
scale distinct, so a dropped term, a wrong sign, a transposed operand or a
wrong scale index all change the result), the all-ones closed form, exact
integer products, and invariances (scale doubling, row permutation, grouped
= per-expert, ROW mode with block-constant scales = BLOCK128 mode).
"""
from fractions import Fraction

import numpy as np
import pytest

from tests import exact


def _codes(rng, shape, lo=0x00, hi=0xFF):
    c = rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    return c


def _scales(rng, shape):
    return (rng.random(shape) * 3 + 0.01).astype(np.float32) * np.float32(2.0 ** -7)


def _exact_entry(qa, sa, qb, sb, mode, m, n):
    K = qa.shape[1]
    c = Fraction(0)
    t = Fraction(0)
    for kb in range(K // 128):
        p = sum((exact.e4m3_value(int(qa[m, k])) * exact.e4m3_value(int(qb[n, k])) for k in range(kb * 128, kb * 128 + 128)), Fraction(0))
        pa = sum((abs(exact.e4m3_value(int(qa[m, k])) * exact.e4m3_value(int(qb[n, k]))) for k in range(kb * 128, kb * 128 + 128)), Fraction(0))
        s_b = sb[n // 128, kb] if mode == 0 else sb[n, kb]
        scl = Fraction(float(sa[m, kb])) * Fraction(float(s_b))
        c += p * scl
        t += pa * abs(scl)
    return c, t


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("K", [128, 384])
def test_gemm_matches_exact_rational(oracle, mode, K):
    rng = np.random.default_rng(K + 10 * mode)
    M, N = 3, 130
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = _scales(rng, (M, K // 128))
    sb = _scales(rng, (2, K // 128)) if mode == 0 else _scales(rng, (N, K // 128))
    pairs = [(0, 0), (1, 1), (2, 129), (0, 128), (2, 3)]
    c, t = oracle.gemm_entries(qa, sa, qb, sb, [m for m, _ in pairs], [n for _, n in pairs], mode)
    for i, (m, n) in enumerate(pairs):
        ce, te = _exact_entry(qa, sa, qb, sb, mode, m, n)
        assert abs(Fraction(c[i]) - ce) <= Fraction(1, 10 ** 14) * te, (m, n)
        assert abs(Fraction(t[i]) - te) <= Fraction(1, 10 ** 14) * te
    # full form agrees with the entry form bitwise
    cf, tf = oracle.gemm(qa, sa, qb, sb, mode)
    for i, (m, n) in enumerate(pairs):
        assert cf[m, n] == c[i] and tf[m, n] == t[i]


def test_gemm_all_ones_closed_form(oracle):
    K = 512
    x = np.ones((4, K), np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qb, sb = oracle.quantize_weight_128x128(np.ones((3, K), np.float32))
    s = np.float32(1.0) / np.float32(448.0)
    assert np.all(qa == 0x7E) and np.all(qb == 0x7E) and np.all(sa == s) and np.all(sb == s)
    c, t = oracle.gemm(qa, sa, qb, sb, 0)
    expected = K * (448 * Fraction(float(s))) ** 2
    assert np.all(np.abs(c - float(expected)) <= 1e-15 * float(expected))
    assert np.all(t == c)


def test_gemm_exact_integer_products(oracle):
    """Codes of small integers with unit scales: every sum is an exact integer,
    so C equals the int64 matrix product."""
    rng = np.random.default_rng(4)
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16], np.float32)
    a = rng.choice(ints, (5, 256)) * rng.choice([-1, 1], (5, 256))
    b = rng.choice(ints, (7, 256)) * rng.choice([-1, 1], (7, 256))
    qa = oracle.e4m3_encode(a.astype(np.float32)).reshape(a.shape)
    qb = oracle.e4m3_encode(b.astype(np.float32)).reshape(b.shape)
    sa = np.ones((5, 2), np.float32)
    sb = np.ones((1, 2), np.float32)
    c, _ = oracle.gemm(qa, sa, qb, sb, 0)
    assert np.array_equal(c, (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64))


def test_gemm_invariances(oracle):
    rng = np.random.default_rng(9)
    M, N, K = 6, 200, 384
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa, sb = _scales(rng, (M, 3)), _scales(rng, (2, 3))
    c, t = oracle.gemm(qa, sa, qb, sb, 0)
    c2, _ = oracle.gemm(qa, sa * np.float32(2), qb, sb, 0)
    assert np.array_equal(c2, 2 * c)
    perm = rng.permutation(M)
    c3, _ = oracle.gemm(qa[perm], sa[perm], qb, sb, 0)
    assert np.array_equal(c3, c[perm])
    # ROW mode with scales constant over each 128-row block == BLOCK128 mode
    sb_row = np.repeat(sb, 128, axis=0)[:N]
    c4, t4 = oracle.gemm(qa, sa, qb, sb_row, 1)
    assert np.array_equal(c4, c) and np.array_equal(t4, t)
    # negating B negates C
    neg = qb ^ np.uint8(0x80)
    c5, _ = oracle.gemm(qa, sa, neg, sb, 0)
    assert np.array_equal(c5, -c)


def test_grouped_equals_per_expert(oracle):
    rng = np.random.default_rng(12)
    counts = np.array([0, 5, 1, 0, 9, 3])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    G, N, K = len(counts), 140, 256
    M = int(off[-1])
    qa, sa = _codes(rng, (M, K)), _scales(rng, (M, 2))
    qb = _codes(rng, (G, N, K))
    sb = _scales(rng, (G, 2, 2))
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c, t = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    c = c.reshape(M, N)
    for g in range(G):
        rows = slice(off[g], off[g + 1])
        if counts[g] == 0:
            continue
        ce, _ = oracle.gemm(qa[rows], sa[rows], qb[g], sb[g], 0)
        assert np.array_equal(c[rows], ce)
    m, n = 7, 139  # one entry against the exact rational
    g = int(np.searchsorted(off, m, side="right") - 1)
    ce, te = _exact_entry(qa, sa, qb[g], sb[g], 0, m, n)
    assert abs(Fraction(c[m, n]) - ce) <= Fraction(1, 10 ** 14) * te


def _exact_dgrad(qdy, sdy, qw, sw, m, k):
    N = qdy.shape[1]
    c = Fraction(0)
    t = Fraction(0)
    for nb in range(N // 128):
        prods = [exact.e4m3_value(int(qdy[m, n])) * exact.e4m3_value(int(qw[n, k])) for n in range(nb * 128, nb * 128 + 128)]
        scl = Fraction(float(sdy[m, nb])) * Fraction(float(sw[nb, k // 128]))
        c += sum(prods, Fraction(0)) * scl
        t += sum((abs(p) for p in prods), Fraction(0)) * abs(scl)
    return c, t


@pytest.mark.parametrize("N", [128, 384])
def test_dgrad_matches_exact_rational(oracle, N):
    """dX = dY W on W's own [N][K] layout: every chunk scale distinct, so a
    transposed operand or a wrong scale index changes the result."""
    rng = np.random.default_rng(N + 3)
    M, K = 3, 260
    qdy, qw = _codes(rng, (M, N)), _codes(rng, (N, K))
    sdy = _scales(rng, (M, N // 128))
    sw = _scales(rng, (N // 128, 3))
    pairs = [(0, 0), (1, 127), (2, 128), (0, 259), (2, 200)]
    c, t = oracle.dgrad_entries(qdy, sdy, qw, sw, [m for m, _ in pairs], [k for _, k in pairs])
    for i, (m, k) in enumerate(pairs):
        ce, te = _exact_dgrad(qdy, sdy, qw, sw, m, k)
        assert abs(Fraction(c[i]) - ce) <= Fraction(1, 10 ** 14) * te, (m, k)
        assert abs(Fraction(t[i]) - te) <= Fraction(1, 10 ** 14) * te


def test_dgrad_is_gemm_with_transposed_weight(oracle):
    """Transposing W's codes and its block-scale matrix turns Dgrad into the
    plain GEMM with the same products in the same order: equal bit for bit.
    Quantizing W^T per 128x128 block gives the transposed codes and scales of
    quantizing W (a block holds the same elements either way)."""
    rng = np.random.default_rng(12)
    M, N, K = 5, 256, 300
    dy = rng.standard_normal((M, N)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qdy, sdy = oracle.quantize_act_1x128(dy)
    qw, sw = oracle.quantize_weight_128x128(w)
    qwt, swt = oracle.quantize_weight_128x128(w.T.copy())
    assert np.array_equal(qwt, qw.T) and np.array_equal(swt, sw.T)
    c1, t1 = oracle.dgrad(qdy, sdy, qw, sw)
    c2, t2 = oracle.gemm(qdy, sdy, qwt, swt, 0)
    assert np.array_equal(c1, c2) and np.array_equal(t1, t2)
