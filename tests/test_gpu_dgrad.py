"""GPU parity of the Dgrad path: the exact weight transpose
(fp8q_transpose_weight) and dX = dY W through the block-scaled GEMM, against
the oracle's Dgrad written on W's own layout."""
import numpy as np
import pytest
import torch

from tests.parity import assert_codes_equal, assert_gemm_close, assert_scales_equal, dev, dev_codes, host_f32, host_u8, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(256, 384), (300, 520), (128, 128), (7, 1000), (1040, 130), (1, 16)])
def test_transpose_weight_exact(fp8q, oracle, shape):
    N, K = shape
    say(f"transpose_weight {shape}")
    rng = np.random.default_rng(N * 3 + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw, sw = oracle.quantize_weight_128x128(w)
    qt, st = fp8q.transpose_weight(dev_codes(qw), dev(sw))
    torch.cuda.synchronize()
    assert_codes_equal(host_u8(qt), qw.T, "transposed codes")
    assert_scales_equal(host_f32(st), sw.T, "transposed scales")


def test_transpose_equals_quantizing_the_transpose(fp8q):
    """On the device alone: transpose(quantize_weight(W)) equals
    quantize_weight(W^T) bit for bit (a 128x128 block has the same elements
    either way)."""
    rng = np.random.default_rng(2)
    w = torch.from_numpy((rng.standard_normal((640, 896)) * 0.02).astype(np.float32)).to(torch.bfloat16).cuda()
    q, s = fp8q.quantize_weight(w)
    qt, st = fp8q.transpose_weight(q, s)
    q2, s2 = fp8q.quantize_weight(w.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(qt.cpu(), q2.cpu()) and torch.equal(st.cpu(), s2.cpu())


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(300, 640, 520), (256, 128, 256), (1, 384, 130), (513, 1024, 300)])
def test_dgrad_parity(fp8q, oracle, shape, out_dtype):
    """dX[M][K] = dY[M][N] W[N][K]; dY ~ N(0, 1e-3) in 1x128 tiles along N."""
    M, N, K = shape
    say(f"dgrad {shape} {out_dtype}")
    rng = np.random.default_rng(M + N + K)
    dy = (rng.standard_normal((M, N)) * 1e-3).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qdy, sdy = oracle.quantize_act_1x128(dy)
    qw, sw = oracle.quantize_weight_128x128(w)
    c_ref, t_ref = oracle.dgrad(qdy, sdy, qw, sw)
    qt, st = fp8q.transpose_weight(dev_codes(qw), dev(sw))
    dx = fp8q.dgrad(dev_codes(qdy), dev(np.ascontiguousarray(sdy.T)), qt, st, out_dtype=out_dtype)
    torch.cuda.synchronize()
    r = assert_gemm_close(host_f32(dx), c_ref, t_ref, out_dtype, f"dgrad {shape}")
    say(f"  worst err/bound = {r:.3f}")


def test_dgrad_full_size(fp8q, oracle):
    """The Linear backward at 4096 tokens x 7168 x 7168 (bf16 dX), checked on
    sampled outputs plus whole rows and columns at tile edges."""
    M, N, K = 4096, 7168, 7168
    say("dgrad full 4096x7168x7168")
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    dy = (torch.randn((M, N), generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qdy, sdy = fp8q.quantize_act(dy)
    qw, sw = fp8q.quantize_weight(w)
    qt, st = fp8q.transpose_weight(qw, sw)
    dx = fp8q.dgrad(qdy, sdy, qt, st)
    torch.cuda.synchronize()
    qdy_o, sdy_o = oracle.quantize_act_1x128(host_f32(dy))
    qw_o, sw_o = oracle.quantize_weight_128x128(host_f32(w))
    assert_codes_equal(host_u8(qdy), qdy_o, "dY codes")
    assert_codes_equal(host_u8(qt), qw_o.T, "W^T codes")
    assert_scales_equal(host_f32(st), sw_o.T, "W^T scales")
    rng = np.random.default_rng(1)
    im = np.concatenate([rng.integers(0, M, 4096), np.full(K, 255), np.arange(M)]).astype(np.int64)
    ik = np.concatenate([rng.integers(0, K, 4096), np.arange(K), np.full(M, 7167)]).astype(np.int64)
    c, t = oracle.dgrad_entries(qdy_o, sdy_o, qw_o, sw_o, im, ik)
    r = assert_gemm_close(host_f32(dx)[im, ik], c, t, torch.bfloat16, "dgrad full")
    say(f"  worst err/bound = {r:.3f}")
