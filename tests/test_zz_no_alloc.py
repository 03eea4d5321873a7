"""fp8q_gemm_splitk_noalloc (split-K with the library's own device scratch,
for callers that cannot allocate) against fp8q_gemm_splitk with a caller
workspace: same slice plan and kernels, so the same bits.  Two calls in a
row, the second on a smaller problem, each checked against the workspace
entry point bit for bit and against the oracle on sampled outputs.  Runs
alone in a fresh process as well as after the other tests."""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu


def _operands(oracle, M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qb, sb = oracle.quantize_weight_128x128(w)
    return qa, sa, qb, sb


def _args(a, sa_d, b, sb_d, M, N, K, c):
    return (a.data_ptr(), a.stride(0), sa_d.data_ptr(), sa_d.stride(0), b.data_ptr(), b.stride(0),
            sb_d.data_ptr(), sb_d.stride(0), 0, M, N, K, c.data_ptr(), 0 if c.dtype == torch.float32 else 1,
            c.stride(0), 0, 0)


@pytest.mark.parametrize("first,second", [((1024, 1024, 65536), (300, 520, 5120))])
def test_noalloc_matches_workspace_entry(fp8q, oracle, first, second):
    stream = torch.cuda.current_stream().cuda_stream
    for M, N, K in (first, second):
        need = fp8q.fp8q_gemm_splitk_workspace(M, N, K)
        say(f"no-alloc split-K {M}x{N}x{K}: plan needs {need} B of {fp8q.SPLITK_SCRATCH_BYTES}")
        assert 0 < need <= fp8q.SPLITK_SCRATCH_BYTES
        qa, sa, qb, sb = _operands(oracle, M, N, K, seed=M + K)
        a, b = dev_codes(qa), dev_codes(qb)
        sa_d, sb_d = dev(np.ascontiguousarray(sa.T)), dev(sb)
        c_ws = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
        base = (ws.data_ptr() + 255) // 256 * 256
        assert fp8q.fp8q_gemm_splitk(*_args(a, sa_d, b, sb_d, M, N, K, c_ws), base, need, stream) == 0
        c_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        st = fp8q.fp8q_gemm_splitk_noalloc(*_args(a, sa_d, b, sb_d, M, N, K, c_na), stream)
        assert st == 0, fp8q.fp8q_strerror(st)
        torch.cuda.synchronize()
        assert torch.equal(c_na, c_ws), "no-alloc result differs from the workspace entry point"
        rng = np.random.default_rng(M)
        im, jn = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
        c, t = oracle.gemm_entries(qa, sa, qb, sb, im, jn, 0)
        r = assert_gemm_close(host_f32(c_na)[im, jn], c, t, torch.float32, f"no-alloc {M}x{N}x{K}")
        say(f"  bitwise equal to the workspace entry point; worst err/bound {r:.3f}")


def test_noalloc_argument_errors(fp8q):
    """Invalid arguments are reported before the scratch is touched."""
    st = fp8q.fp8q_gemm_splitk_noalloc(0, 65536, 0, 1024, 0, 65536, 0, 512, 0, 1024, 1024, 65536, 0, 0, 1024,
                                       0, 0, None)
    assert st == fp8q.FP8Q_EINVAL
    st = fp8q.fp8q_gemm_splitk_noalloc(1 << 20, 65536, 1 << 20, 1024, 1 << 20, 65536, 1 << 20, 512, 0, 1024, 1024,
                                       65536 + 64, 1 << 20, 0, 1024, 0, 0, None)
    assert st == fp8q.FP8Q_ESHAPE
