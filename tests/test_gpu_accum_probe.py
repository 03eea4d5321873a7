"""Accumulation precision of the gfx950 matrix cores, measured through the
library's two GEMM datapaths (fp8q_gemm_ex flags).

The pages report that FP8 tensor cores keep only about 14 bits while adding
products (page 3, why-be.why-be.co.kr wr_id=55081, passage on limited
accumulation precision and Figure 7(b)).  These tests pin what gfx950 does:

* default datapath (f16 matrix instructions on exactly converted codes): the
  products of one chunk add like FP32, so a small product next to a large one
  survives;
* FP8Q_GEMM_MMA_FP8 (native FP8 matrix instruction): each run of 8 adjacent
  K products is added inside a window of about 14 binary orders below the
  run's largest product; bits below it are truncated toward zero.  Products
  in different runs add like FP32.

Inputs are hand-built codes with unit scales, so every expected value is an
exact fp32 number: 256 = 16 * 16 is the large product, 2^-6 = 2^-3 * 2^-3 and
2^-5 = 2^-2 * 2^-3 the small ones.
"""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu

C16, C2M3, C2M2, CN2M3 = 0x58, 0x20, 0x28, 0xA0  # E4M3 codes of 16, 2^-3, 2^-2, -2^-3


def _gemm(fp8q, qa, qb, flags):
    M, K = qa.shape
    N = qb.shape[0]
    sa = dev(np.ones((K // 128, M), np.float32))
    sb = dev(np.ones((-(-N // 128), K // 128), np.float32))
    out = fp8q.gemm(dev_codes(qa), sa, dev_codes(qb), sb, out_dtype=torch.float32, flags=flags)
    torch.cuda.synchronize()
    return host_f32(out).astype(np.float64)


def test_small_product_beside_large_one_at_every_k(fp8q):
    """Row k (1 <= k < 128) holds the product 256 at K index 0 and 2^-6 at K
    index k.  The exact sum is 256 + 2^-6 for every row; the FP8 instruction
    drops 2^-6 (14 orders below 256) exactly when k is in the first run of 8."""
    K, N = 128, 16
    rows = np.arange(1, K)
    qa = np.zeros((K - 1, K), np.uint8)
    qa[:, 0] = C16
    qa[rows - 1, rows] = C2M3
    qb = np.full((N, K), C2M3, np.uint8)
    qb[:, 0] = C16
    say("probe: 256 + 2^-6 at every K position")
    exact = 256.0 + 2.0 ** -6
    got_f16 = _gemm(fp8q, qa, qb, 0)
    assert np.all(got_f16 == exact)
    got_fp8 = _gemm(fp8q, qa, qb, fp8q.FP8Q_GEMM_MMA_FP8)
    expect = np.where(rows < 8, 256.0, exact)[:, None] * np.ones((1, N))
    assert np.array_equal(got_fp8, expect), np.unique(got_fp8, return_counts=True)


def test_window_edge_and_truncation_sign(fp8q):
    """Inside one run of 8: 2^-5 (13 orders below 256) is kept, 2^-6 is
    dropped, and -2^-6 is dropped too (truncation toward zero, not rounding
    to nearest, which would give 256 - 2^-6 or 256)."""
    K, N = 128, 16
    qa = np.zeros((3, K), np.uint8)
    qa[:, 0] = C16
    qa[0, 1] = C2M2   # 2^-2 * 2^-3 = 2^-5
    qa[1, 1] = C2M3   # 2^-6
    qa[2, 1] = CN2M3  # -2^-6
    qb = np.full((N, K), C2M3, np.uint8)
    qb[:, 0] = C16
    say("probe: window edge and sign")
    got_f16 = _gemm(fp8q, qa, qb, 0)
    assert np.all(got_f16[:, 0] == [256 + 2.0 ** -5, 256 + 2.0 ** -6, 256 - 2.0 ** -6])
    got_fp8 = _gemm(fp8q, qa, qb, fp8q.FP8Q_GEMM_MMA_FP8)
    assert np.all(got_fp8[:, 0] == [256 + 2.0 ** -5, 256.0, 256.0])


def test_promotion_keeps_each_chunk(fp8q):
    """The chunk partials are promoted into an FP32 total: a chunk whose only
    product is 2^-6 still counts fully after a chunk of 256 on both paths."""
    K, N = 256, 16
    qa = np.zeros((1, K), np.uint8)
    qa[0, 0] = C16
    qa[0, 128] = C2M3
    qb = np.full((N, K), C2M3, np.uint8)
    qb[:, 0] = C16
    for flags in (0, fp8q.FP8Q_GEMM_MMA_FP8):
        assert np.all(_gemm(fp8q, qa, qb, flags) == 256.0 + 2.0 ** -6)


@pytest.mark.parametrize("mode", [0, 1])
def test_fp8_datapath_within_its_bound(fp8q, oracle, mode):
    """On fprop-like data (Student-t activations, N(0, 0.02) weights) the FP8
    datapath stays within 2^-10 * T plus the default bound; the worst ratio
    err / T is reported next to the default datapath's."""
    M, N, K = 300, 520, 1024
    rng = np.random.default_rng(11 + mode)
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    if mode == 0:
        qb, sb = oracle.quantize_weight_128x128(w)
        sb_dev = sb
    else:
        qbt, sbt = oracle.quantize_act_128x1(w.T.copy())
        qb, sb, sb_dev = qbt.T.copy(), sbt.T.copy(), sbt
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, mode)
    worst = {}
    for flags in (0, fp8q.FP8Q_GEMM_MMA_FP8):
        out = fp8q.gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev_codes(qb),
                        dev(np.ascontiguousarray(sb_dev)), bscale=mode, out_dtype=torch.float32,
                        flags=flags)
        torch.cuda.synchronize()
        got = host_f32(out).astype(np.float64)
        err = np.abs(got - c_ref)
        worst[flags] = float((err / t_ref).max())
        if flags == 0:
            assert_gemm_close(got, c_ref, t_ref, torch.float32, "default datapath")
        else:
            assert np.all(err <= 2.0 ** -10 * t_ref + 1e-5 * t_ref)
    say(f"  max err/T: default {worst[0]:.2e}, fp8 datapath {worst[fp8q.FP8Q_GEMM_MMA_FP8]:.2e}")


def test_grouped_fp8_datapath(fp8q, oracle):
    counts, N, K = [0, 37, 300, 129], 384, 512
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(3)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    say("grouped fp8 datapath")
    out = fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                            out_dtype=torch.float32, flags=fp8q.FP8Q_GEMM_MMA_FP8)
    torch.cuda.synchronize()
    err = np.abs(host_f32(out).astype(np.float64) - c_ref.reshape(M, N))
    assert np.all(err <= (2.0 ** -10 + 1e-5) * t_ref.reshape(M, N))
