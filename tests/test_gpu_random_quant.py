"""Seeded sweep of quantizer, requantization, weight-transpose and gather
shapes against the CPU oracle, bit for bit.

Each case draws rows and columns (1..600, any residue modulo 128), the input
dtype, the scale rule (fp32 or power-of-two), the value distribution and a
padded row stride, and checks every code and scale of:
  - quantize_act 1x128 and 128x1 (transposed output),
  - quantize_weight 128x128,
  - requant_transpose of the oracle's own 1x128 codes,
  - transpose_weight of the oracle's own 128x128 codes (an exact permutation),
  - gather_quantize_act with repeated, permuted and out-of-range row indices.
"""
import numpy as np
import pytest
import torch

from tests.parity import assert_codes_equal, assert_scales_equal, dev, dev_codes, host_f32, host_u8, say
from tests.test_gpu_quantize import _padded

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(5000 + seed)
    rows = int(rng.integers(1, 601))
    cols = int(rng.integers(1, 601))
    dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    mode = int(rng.integers(0, 2))
    kind = ["t", "n", "wide"][int(rng.integers(0, 3))]
    if kind == "t":
        x = rng.standard_t(3, (rows, cols)).astype(np.float32)
    elif kind == "n":
        x = rng.standard_normal((rows, cols)).astype(np.float32)
    else:
        e = rng.integers(-140, 30, size=(rows, cols))
        x = (rng.choice([-1.0, 1.0], (rows, cols)) * rng.random((rows, cols)) * np.exp2(e)).astype(np.float32)
    x[rng.integers(0, rows), :] = 0.0
    t = torch.from_numpy(x).to(dtype)
    return rng, rows, cols, dtype, mode, kind, t


@pytest.mark.parametrize("seed", range(16))
def test_random_quantizers(fp8q, oracle, seed):
    rng, rows, cols, dtype, mode, kind, t = _draw(seed)
    say(f"random quantizers seed={seed} {rows}x{cols} {dtype} mode={mode} {kind}")
    xh = host_f32(t)  # exact widening of the input the GPU sees
    xd = _padded(t, 8 if dtype == torch.bfloat16 else 4)

    q, s = fp8q.quantize_act(xd, fp8q.FP8Q_TILE_1x128, scale_mode=mode)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_1x128(xh, mode)
    assert_codes_equal(host_u8(q), qo, "1x128 codes")
    assert_scales_equal(host_f32(s), so.T, "1x128 scales")

    q, s = fp8q.quantize_act(xd, fp8q.FP8Q_TILE_128x1, scale_mode=mode)
    torch.cuda.synchronize()
    qo2, so2 = oracle.quantize_act_128x1(xh, mode)
    assert_codes_equal(host_u8(q), qo2.T, "128x1 codes")
    assert_scales_equal(host_f32(s), so2, "128x1 scales")

    q, s = fp8q.quantize_weight(xd, scale_mode=mode)
    torch.cuda.synchronize()
    qw, sw = oracle.quantize_weight_128x128(xh, mode)
    assert_codes_equal(host_u8(q), qw, "128x128 codes")
    assert_scales_equal(host_f32(s), sw, "128x128 scales")

    qt, st = fp8q.requant_transpose(dev_codes(qo), dev(np.ascontiguousarray(so.T)), scale_mode=mode)
    torch.cuda.synchronize()
    qr, sr = oracle.requant_1x128_to_128x1(qo, so, mode)
    assert_codes_equal(host_u8(qt), qr.T, "requant codes")
    assert_scales_equal(host_f32(st), sr, "requant scales")

    qwt, swt = fp8q.transpose_weight(dev_codes(qw), dev(sw))
    torch.cuda.synchronize()
    assert_codes_equal(host_u8(qwt), np.ascontiguousarray(qw.T), "transposed weight codes")
    assert_scales_equal(host_f32(swt), np.ascontiguousarray(sw.T), "transposed weight scales")

    n_out = int(rng.integers(1, 2 * rows + 2))
    idx = rng.integers(-2, rows + 2, n_out).astype(np.int32)  # some indices outside the input
    qg, sg = fp8q.gather_quantize_act(xd, torch.from_numpy(idx).cuda(), scale_mode=mode)
    torch.cuda.synchronize()
    qgo, sgo = oracle.gather_quantize_act_1x128(xh, idx, mode)
    assert_codes_equal(host_u8(qg), qgo, "gather codes")
    assert_scales_equal(host_f32(sg), sgo.T, "gather scales")
