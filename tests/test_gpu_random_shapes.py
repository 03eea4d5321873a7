"""Seeded sweep of GEMM shapes, output strides and output offsets against the
FP64 oracle.

Each case draws M, N (1..700), K (128..1024, a multiple of 128), the B-scale
mode, the output dtype, accumulate (fp32 only), and places C inside a larger
buffer at a random row stride and column offset.  That exercises the rows
read past the matrix (they must contribute nothing), the 16-byte output path
(taken when C and its row stride are 16-byte aligned) and the element-store
path (taken otherwise; even seeds force an aligned C), on full and ragged tiles.  Every output element is
checked to the tolerance of tests/parity.py, and the padding around C must be
untouched.
"""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.integers(1, 701))
    N = int(rng.integers(1, 701))
    K = 128 * int(rng.integers(1, 9))
    mode = int(rng.integers(0, 2))
    f32 = bool(rng.integers(0, 2))
    acc = f32 and bool(rng.integers(0, 2))
    pad = int(rng.integers(0, 40))      # extra row-stride elements
    col0 = int(rng.integers(0, 9))      # column offset of C inside its buffer
    if seed % 2 == 0:                   # 16-byte aligned C and row stride
        col0 = 8 * (col0 % 2)
        pad += (-(N + col0 + pad)) % 8
    return rng, M, N, K, mode, f32, acc, pad, col0


@pytest.mark.parametrize("seed", range(24))
def test_random_gemm(fp8q, oracle, seed):
    rng, M, N, K, mode, f32, acc, pad, col0 = _case(seed)
    dt = torch.float32 if f32 else torch.bfloat16
    say(f"random gemm seed={seed} M={M} N={N} K={K} mode={mode} {dt} acc={acc} pad={pad} col0={col0}")
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

    ldc = N + col0 + pad
    sentinel = -7.0
    buf = torch.full((M + 1, ldc), sentinel, dtype=dt, device="cuda")
    c = buf[:M, col0:col0 + N]
    c0 = None
    if acc:
        c0 = rng.standard_normal((M, N)).astype(np.float32)
        c.copy_(torch.from_numpy(c0).cuda())
    fp8q.gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev_codes(qb), dev(np.ascontiguousarray(sb_dev)),
              bscale=mode, out_dtype=dt, c=c, accumulate=acc)
    torch.cuda.synchronize()
    got = host_f32(c)
    if acc:
        # C += result: the fp32 addition adds at most half an fp32 ulp of the sum
        exp = c0.astype(np.float64) + c_ref
        err = np.abs(got.astype(np.float64) - exp)
        bound = 1e-5 * t_ref + np.abs(exp) * 2.0 ** -24 + 1e-30
        assert np.all(err <= bound), f"{int((err > bound).sum())} outputs beyond the bound"
    else:
        assert_gemm_close(got, c_ref, t_ref, dt, f"random gemm {seed}")
    host = host_f32(buf)
    mask = np.ones(host.shape, bool)
    mask[:M, col0:col0 + N] = False
    assert np.all(host[mask] == sentinel), "GEMM wrote outside C"


def _grouped_case(seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.integers(1, 25))
    counts = rng.integers(0, 301, G)
    counts[rng.random(G) < 0.2] = 0          # some experts receive no rows
    if counts.sum() == 0:
        counts[0] = 1
    N = int(rng.integers(1, 521))
    K = 128 * int(rng.integers(1, 5))
    f32 = bool(rng.integers(0, 2))
    pad = int(rng.integers(0, 24))            # extra row-stride elements of C
    return rng, counts.astype(np.int64), N, K, f32, pad


@pytest.mark.parametrize("seed", range(12))
def test_random_grouped(fp8q, oracle, seed):
    """Seeded sweep of grouped GEMMs: 1..24 experts with 0..300 rows each
    (about a fifth empty), N in 1..520 (ragged last column tile and weight
    block), K up to 512, fp32 or bf16 output in a wider buffer.  Every output
    row against the oracle's per-expert product; the padding columns and the
    guard row after C stay untouched."""
    rng, counts, N, K, f32, pad = _grouped_case(seed)
    G = counts.size
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    dt = torch.float32 if f32 else torch.bfloat16
    say(f"random grouped seed={seed} G={G} M={M} N={N} K={K} {dt} pad={pad}")
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    sentinel = -7.0
    buf = torch.full((M + 1, N + pad), sentinel, dtype=dt, device="cuda")
    c = buf[:M, :N]
    fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off), c=c)
    torch.cuda.synchronize()
    got = host_f32(buf)
    assert_gemm_close(got[:M, :N], c_ref.reshape(M, N), t_ref.reshape(M, N), dt, f"grouped seed {seed}")
    assert np.all(got[:M, N:] == sentinel), "padding columns written"
    assert np.all(got[M] == sentinel), "guard row written"
