"""The tensor helpers refuse arguments the C ABI cannot see through: wrong
scale layouts (which the ABI's leading-dimension checks may accept), wrong
dtypes, mismatched shapes and host tensors.  All checks run before the
library is called, so these tests need no GPU."""
import pytest
import torch

import fp8_fine_grained_x128_amd as fp8q

M, N, K = 256, 1024, 512


def _ops():
    a = torch.zeros((M, K), dtype=torch.uint8)
    b = torch.zeros((N, K), dtype=torch.uint8)
    sa = torch.zeros((K // 128, M), dtype=torch.float32)
    sb_block = torch.zeros((N // 128, K // 128), dtype=torch.float32)
    sb_row = torch.zeros((K // 128, N), dtype=torch.float32)
    return a, b, sa, sb_block, sb_row


def test_gemm_rejects_row_scales_in_block_mode():
    """ROW-layout B scales [K/128][N] passed with BLOCK128: the ABI's
    ldsb >= K/128 check would accept them (ldsb = N), and the kernel would
    read scale rows past the allocation."""
    a, b, sa, _, sb_row = _ops()
    with pytest.raises(ValueError, match="BLOCK128"):
        fp8q.gemm(a, sa, b, sb_row, bscale=fp8q.FP8Q_BSCALE_BLOCK128)


def test_gemm_rejects_block_scales_in_row_mode():
    a, b, sa, sb_block, _ = _ops()
    with pytest.raises(ValueError, match="ROW"):
        fp8q.gemm(a, sa, b, sb_block, bscale=fp8q.FP8Q_BSCALE_ROW)


def test_gemm_rejects_transposed_activation_scales():
    a, b, _, sb_block, _ = _ops()
    with pytest.raises(ValueError, match="s_a"):
        fp8q.gemm(a, torch.zeros((M, K // 128), dtype=torch.float32), b, sb_block)


def test_gemm_rejects_wrong_dtypes_and_shapes():
    a, b, sa, sb_block, _ = _ops()
    with pytest.raises(ValueError, match="1-byte"):
        fp8q.gemm(a.float(), sa, b, sb_block)
    with pytest.raises(ValueError, match="float32"):
        fp8q.gemm(a, sa.double(), b, sb_block)
    with pytest.raises(ValueError, match="must be"):
        fp8q.gemm(a, sa, b[:, :256], sb_block)


def test_host_tensors_are_refused():
    a, b, sa, sb_block, _ = _ops()
    with pytest.raises(ValueError, match="HIP device"):
        fp8q.gemm(a, sa, b, sb_block)
    with pytest.raises(ValueError, match="HIP device"):
        fp8q.quantize_act(torch.zeros((4, 128)))
    with pytest.raises(ValueError, match="HIP device"):
        fp8q.quantize_weight(torch.zeros((128, 128)))


def test_grouped_and_requant_layouts():
    a = torch.zeros((300, K), dtype=torch.uint8)
    sa = torch.zeros((K // 128, 300), dtype=torch.float32)
    b = torch.zeros((4, N, K), dtype=torch.uint8)
    off = torch.zeros(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="s_b"):
        fp8q.grouped_gemm(a, sa, b, torch.zeros((4, K // 128, N // 128)), off)
    with pytest.raises(ValueError, match="requant_transpose scales"):
        fp8q.requant_transpose(a, torch.zeros((300, K // 128), dtype=torch.float32))
