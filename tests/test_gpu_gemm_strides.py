"""GPU parity of the GEMMs at the largest accepted operand row stride.

The kernels reach a tile's operand rows through a buffer descriptor whose
record count is (valid rows) x (row stride) and whose offsets are 32-bit; the
API accepts row strides below 2^24, so a 256-row tile spans almost 2^32 bytes.
These tests place A (or B) rows 2^24 - 16 bytes apart (a 5 GB allocation of
which only the first K bytes of each row are written) and check the result
against the FP64 oracle and bit for bit against the same GEMM on compact
operands.
"""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu
BIG_LD = (1 << 24) - 16


def _wide(q: np.ndarray) -> torch.Tensor:
    rows, cols = q.shape
    buf = torch.empty((rows, BIG_LD), dtype=torch.uint8, device="cuda")
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    return buf[:, :cols]


def _operands(oracle, M, N, K, seed):
    rng = np.random.default_rng(seed)
    qa, sa = oracle.quantize_act_1x128(rng.standard_normal((M, K)).astype(np.float32))
    qb, sb = oracle.quantize_weight_128x128((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    return qa, sa, qb, sb


@pytest.mark.parametrize("wide", ["a", "b"])
def test_max_row_stride(fp8q, oracle, wide):
    M, N, K = 300, 260, 256
    qa, sa, qb, sb = _operands(oracle, M, N, K, seed=11)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, 0)
    sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(sb)
    say(f"gemm with row stride {BIG_LD} on operand {wide}")
    a_d = _wide(qa) if wide == "a" else dev_codes(qa)
    b_d = _wide(qb) if wide == "b" else dev_codes(qb)
    assert (a_d if wide == "a" else b_d).stride(0) == BIG_LD
    got = fp8q.gemm(a_d, sa_d, b_d, sb_d, out_dtype=torch.float32)
    compact = fp8q.gemm(dev_codes(qa), sa_d, dev_codes(qb), sb_d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, compact)
    assert_gemm_close(host_f32(got), c_ref, t_ref, torch.float32, "wide-stride gemm")
    del a_d, b_d
    torch.cuda.empty_cache()


def test_max_row_stride_grouped(fp8q, oracle):
    counts, N, K = [100, 0, 200], 256, 256
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(12)
    qa, sa = oracle.quantize_act_1x128(rng.standard_normal((M, K)).astype(np.float32))
    qbs, sbs = zip(*[oracle.quantize_weight_128x128((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
                     for _ in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    say(f"grouped gemm with A row stride {BIG_LD}")
    a_d = _wide(qa)
    got = fp8q.grouped_gemm(a_d, dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host_f32(got), c_ref.reshape(M, N), t_ref.reshape(M, N), torch.float32, "wide grouped")
    del a_d
    torch.cuda.empty_cache()
