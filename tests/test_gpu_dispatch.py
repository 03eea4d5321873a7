"""GPU parity of the fused gather + 1x128 quantization (FP8 MoE dispatch)
against the oracle: bit-exact codes and scales for repeated rows, empty slots
(-1 and out-of-range indices), ragged widths, both scale rules; then the
dispatched rows through the grouped GEMM."""
import numpy as np
import pytest
import torch

from fp8_fine_grained_x128_amd import workloads as W
from tests.parity import assert_codes_equal, assert_gemm_close, assert_scales_equal, dev, host_f32, host_u8, say
from tests.test_gpu_quantize import _inputs, _padded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scale_mode", [0, 1])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 1000, 700), (64, 7168, 257), (5, 7, 40), (1, 128, 1)])
def test_gather_quantize_parity(fp8q, oracle, shape, dtype, scale_mode):
    rows_in, cols, rows_out = shape
    say(f"gather_quantize {shape} {dtype} mode={scale_mode}")
    x = _inputs(rows_in, cols, dtype, seed=rows_in + cols + rows_out, kind="t")
    rng = np.random.default_rng(rows_out)
    idx = rng.integers(0, rows_in, rows_out).astype(np.int32)
    if rows_out > 4:
        idx[1] = -1
        idx[3] = rows_in        # out of range: empty slot
        idx[4] = idx[0]         # repeat
    q, s = fp8q.gather_quantize_act(_padded(x, 8 if dtype == torch.bfloat16 else 4), dev(idx),
                                    scale_mode=scale_mode)
    torch.cuda.synchronize()
    qo, so = oracle.gather_quantize_act_1x128(host_f32(x), idx, scale_mode)
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so.T, "scales")


def test_dispatch_then_grouped_gemm(fp8q, oracle):
    """Dispatch 2048 tokens to 16 experts (Zipf counts over 4096 slots),
    quantize in the same pass, and run the grouped GEMM on the dispatched
    codes; outputs checked against the oracle on the oracle's own dispatch."""
    d = W.make_dispatch(2048, 4096, 16, 512, seed=3)
    rng = np.random.default_rng(5)
    N = 384
    w = (rng.standard_normal((16, N, 512)) * 0.02).astype(np.float32)
    qa, sa = fp8q.gather_quantize_act(d.x.cuda(), dev(d.row_index))
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(16)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    y = fp8q.grouped_gemm(qa, sa, dev(qb), dev(sb), dev(d.offsets), out_dtype=torch.float32)
    torch.cuda.synchronize()
    qao, sao = oracle.gather_quantize_act_1x128(host_f32(d.x), d.row_index)
    assert_codes_equal(host_u8(qa), qao, "dispatched codes")
    assert_scales_equal(host_f32(sa), sao.T, "dispatched scales")
    mm, nn = np.meshgrid(np.arange(4096), np.arange(N), indexing="ij")
    c, t = oracle.grouped_gemm_entries(qao, sao, qb, sb, d.offsets, mm.ravel(), nn.ravel())
    assert_gemm_close(host_f32(y), c.reshape(4096, N), t.reshape(4096, N), torch.float32, "dispatch+grouped")


def test_dispatch_full_size(fp8q, oracle):
    """The full dispatch workload (16384 tokens x 7168 -> 32768 expert rows),
    every code and scale checked."""
    d = W.dispatch()
    say("dispatch full 16384 -> 32768 x 7168")
    q, s = fp8q.gather_quantize_act(d.x.cuda(), dev(d.row_index))
    torch.cuda.synchronize()
    qo, so = oracle.gather_quantize_act_1x128(host_f32(d.x), d.row_index)
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so.T, "scales")
