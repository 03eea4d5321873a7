"""GPU parity of the power-of-two scale quantizers (FP8Q_SCALE_POW2) against
the oracle: codes and scales bit-exact on ragged shapes spanning several
tiles, edge rows (zeros, signed zeros, subnormal and wide-range data, exact
multiples of 448) and the requantization chain."""
import numpy as np
import pytest
import torch

from tests.parity import assert_codes_equal, assert_scales_equal, dev, dev_codes, host_f32, host_u8, say
from tests.test_gpu_quantize import _inputs, _padded

pytestmark = pytest.mark.gpu
POW2 = 1


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 128), (5, 7), (300, 1000), (257, 1032), (64, 7168)])
@pytest.mark.parametrize("kind", ["t", "wide"])
def test_quantize_act_1x128_pow2(fp8q, oracle, dtype, shape, kind):
    rows, cols = shape
    say(f"pow2 quantize_act 1x128 {dtype} {shape} {kind}")
    x = _inputs(rows, cols, dtype, seed=rows * 29 + cols, kind=kind)
    q, s = fp8q.quantize_act(_padded(x, 8 if dtype == torch.bfloat16 else 4), fp8q.FP8Q_TILE_1x128,
                             scale_mode=fp8q.FP8Q_SCALE_POW2)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_1x128(host_f32(x), POW2)
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so.T, "scales")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 200), (1000, 257), (7, 5), (129, 4096)])
def test_quantize_act_128x1_pow2(fp8q, oracle, dtype, shape):
    rows, cols = shape
    say(f"pow2 quantize_act 128x1 {dtype} {shape}")
    x = _inputs(rows, cols, dtype, seed=rows * 13 + cols, kind="wide")
    q, s = fp8q.quantize_act(_padded(x, 8 if dtype == torch.bfloat16 else 4), fp8q.FP8Q_TILE_128x1,
                             scale_mode=fp8q.FP8Q_SCALE_POW2)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_128x1(host_f32(x), POW2)
    assert_codes_equal(host_u8(q), qo.T, "codes (transposed)")
    assert_scales_equal(host_f32(s), so, "scales")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 1000), (256, 7168), (129, 131)])
def test_quantize_weight_pow2(fp8q, oracle, dtype, shape):
    N, K = shape
    say(f"pow2 quantize_weight {dtype} {shape}")
    w = _inputs(N, K, dtype, seed=N + 5 * K, kind="wide" if N == 129 else "n")
    q, s = fp8q.quantize_weight(_padded(w, 8 if dtype == torch.bfloat16 else 4),
                                scale_mode=fp8q.FP8Q_SCALE_POW2)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_weight_128x128(host_f32(w), POW2)
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so, "scales")


@pytest.mark.parametrize("shape", [(300, 1000), (256, 256), (129, 1040)])
def test_requant_transpose_pow2(fp8q, oracle, shape):
    rows, cols = shape
    say(f"pow2 requant_transpose {shape}")
    x = host_f32(_inputs(rows, cols, torch.bfloat16, seed=rows + 3 * cols, kind="wide"))
    q1, s1 = oracle.quantize_act_1x128(x, POW2)
    q2, s2 = oracle.requant_1x128_to_128x1(q1, s1, POW2)
    qt, st = fp8q.requant_transpose(dev_codes(q1), dev(np.ascontiguousarray(s1.T)),
                                    scale_mode=fp8q.FP8Q_SCALE_POW2)
    torch.cuda.synchronize()
    assert_codes_equal(host_u8(qt), q2.T, "codes (transposed)")
    assert_scales_equal(host_f32(st), s2, "scales")


def test_pow2_scale_boundaries(fp8q, oracle):
    """Tiles whose amax sits on both sides of 1.75 * 2^E (the mantissa bound
    0x600000 of the closed form), at powers of two, and in the subnormal
    range, in fp32."""
    rng = np.random.default_rng(8)
    E = rng.integers(-149, 127, size=256)
    mant = np.array([0x600000, 0x600001, 0x5FFFFF, 0, 1, 0x7FFFFF] * 43)[:256]
    bits = np.where(E >= -126, ((E + 127) << 23) | mant, mant | 1).astype(np.uint32)
    amax = bits.view(np.float32)
    x = (rng.standard_normal((256, 128)).astype(np.float32) * 0.001) * amax[:, None]
    x[:, 0] = amax
    q, s = fp8q.quantize_act(dev(x), scale_mode=fp8q.FP8Q_SCALE_POW2)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_1x128(x, POW2)
    assert_scales_equal(host_f32(s), so.T, "scales")
    assert_codes_equal(host_u8(q), qo, "codes")
