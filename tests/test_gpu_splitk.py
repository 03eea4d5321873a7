"""GPU parity of the split-K GEMM (fp8q_gemm_splitk) against the FP64 oracle.

The K chunks are dealt to slices whose FP32 partials are added in slice
order; every output must meet the bound of the datapath, a repeated call
must give the same bits, and nothing outside C and the stated workspace
bytes may be written.  Operands are quantized by the oracle."""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu


def _operands(oracle, M, N, K, mode, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    if mode == 0:
        qb, sb = oracle.quantize_weight_128x128(w)
        sb_dev = sb
    else:
        qb, sbt = oracle.quantize_act_128x1(w.T.copy())
        qb = qb.T.copy()
        sb = sbt.T.copy()
        sb_dev = sbt
    return qa, sa, qb, sb, sb_dev


def _call(fp8q, a, sa_d, b, sb_d, mode, M, N, K, c, flags=0, accumulate=0, ws_extra=0):
    """Raw C-ABI call with a workspace of exactly the queried size (plus a
    guard region filled with a pattern that must survive)."""
    need = fp8q.fp8q_gemm_splitk_workspace(M, N, K)
    ws = torch.full((need + 256 + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    off = base - ws.data_ptr()
    st = fp8q.fp8q_gemm_splitk(a.data_ptr(), a.stride(0), sa_d.data_ptr(), sa_d.stride(0), b.data_ptr(),
                               b.stride(0), sb_d.data_ptr(), sb_d.stride(0), mode, M, N, K, c.data_ptr(),
                               0 if c.dtype == torch.float32 else 1, c.stride(0), accumulate, flags,
                               base if need else 0, need + ws_extra,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, fp8q.fp8q_strerror(st)
    torch.cuda.synchronize()
    guard = ws[off + need:off + need + 4096].cpu().numpy()
    assert np.all(guard == 0x5A), "split-K wrote past its workspace"
    return need


SHAPES = [
    (300, 520, 5120),   # 6 tiles, 40 chunks: 10 slices of 4
    (1, 1000, 8192),    # one ragged tile, 64 chunks: 16 slices
    (257, 130, 2048),   # 2 tiles ragged both ways, 16 chunks: 4 slices
    (1024, 256, 4096),  # 4 full tiles, 32 chunks: 8 slices
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_splitk_parity(fp8q, oracle, mode, out_dtype, shape):
    M, N, K = shape
    say(f"splitk mode={mode} {out_dtype} {shape}")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, mode, seed=M + N + K + mode)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, mode)
    a, b = dev_codes(qa), dev_codes(qb)
    sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(np.ascontiguousarray(sb_dev))
    # C inside a wider buffer: the columns past N must stay untouched
    ldc = N + 8
    buf = torch.full((M, ldc), 7.0, dtype=out_dtype, device="cuda")
    c = buf[:, :N]
    need = _call(fp8q, a, sa_d, b, sb_d, mode, M, N, K, c)
    assert need > 0, "shape expected to split"
    r = assert_gemm_close(host_f32(c), c_ref, t_ref, out_dtype, f"splitk {shape}")
    assert np.all(host_f32(buf[:, N:]) == 7.0)
    say(f"  workspace {need} B, worst err/bound {r:.3f}")
    # deterministic: the slices are added in a fixed order
    c2 = torch.empty((M, N), dtype=out_dtype, device="cuda")
    _call(fp8q, a, sa_d, b, sb_d, mode, M, N, K, c2)
    assert torch.equal(c2, c)


def test_splitk_accumulate_and_binding(fp8q, oracle):
    """accumulate adds to C; the tensor helper gemm() takes the split path by
    itself for such shapes and gives the same bits as the raw call."""
    M, N, K = 300, 520, 5120
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, 0, seed=3)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, 0)
    a, b = dev_codes(qa), dev_codes(qb)
    sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(np.ascontiguousarray(sb_dev))
    base = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    c = dev(base)
    _call(fp8q, a, sa_d, b, sb_d, 0, M, N, K, c, accumulate=1)
    got = host_f32(c).astype(np.float64)
    exp = base.astype(np.float64) + c_ref
    assert np.all(np.abs(got - exp) <= 1e-5 * t_ref + np.abs(exp) * 2.0 ** -24 + 1e-30)
    c1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _call(fp8q, a, sa_d, b, sb_d, 0, M, N, K, c1)
    c2 = fp8q.gemm(a, sa_d, b, sb_d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    # and the unsplit kernel meets the same bound on the same operands
    c3 = fp8q.gemm(a, sa_d, b, sb_d, out_dtype=torch.float32, split_k=False)
    torch.cuda.synchronize()
    assert_gemm_close(host_f32(c3), c_ref, t_ref, torch.float32, "unsplit")


def test_splitk_fp8_datapath(fp8q, oracle):
    """The native FP8 instruction through the split path keeps its own bound
    (2^-10 * T on top of the default one)."""
    M, N, K = 300, 520, 5120
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, 0, seed=4)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, 0)
    a, b = dev_codes(qa), dev_codes(qb)
    sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(np.ascontiguousarray(sb_dev))
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _call(fp8q, a, sa_d, b, sb_d, 0, M, N, K, c, flags=fp8q.FP8Q_GEMM_MMA_FP8)
    err = np.abs(host_f32(c).astype(np.float64) - c_ref)
    assert np.all(err <= (1e-5 + 2.0 ** -10) * t_ref)


def test_splitk_no_split_shape_ignores_workspace(fp8q, oracle):
    """A shape whose tiles fill more than half the GPU, or a K too short to
    split, needs no workspace; the call runs the plain
    kernel (workspace NULL is then valid)."""
    assert fp8q.fp8q_gemm_splitk_workspace(4096, 4096, 1024) == 0  # 256 tiles
    K = 512  # 4 chunks: too short to split at any tile count
    assert fp8q.fp8q_gemm_splitk_workspace(300, 300, K) == 0
    qa, sa, qb, sb, sb_dev = _operands(oracle, 300, 300, K, 0, seed=6)
    a, b = dev_codes(qa), dev_codes(qb)
    sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(np.ascontiguousarray(sb_dev))
    c = torch.empty((300, 300), dtype=torch.float32, device="cuda")
    need = _call(fp8q, a, sa_d, b, sb_d, 0, 300, 300, K, c)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, 0)
    assert need == 0
    assert_gemm_close(host_f32(c), c_ref, t_ref, torch.float32, "300x300x512")
