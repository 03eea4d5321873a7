"""Every entry point under HIP graph capture.

The library makes no allocation, memset or host synchronisation of its own,
so a training step built from it can be captured once and replayed.  One
graph holds the forward pass (quantize X per 1x128, W per 128x128, GEMM), the
backward pass (dY per 1x128 and 128x1, X requantized to 128x1, Wgrad with ROW
scales, W transposed, Dgrad) and an MoE dispatch + grouped GEMM.  The graph is
replayed several times, with eager library work and synchronisations in
between and new values copied into its inputs, and each replay's outputs must
equal the eager results on the same inputs bit for bit (every output element
is computed by one wave in a fixed order, so eager runs are deterministic).
"""
import numpy as np
import pytest
import torch

from fp8_fine_grained_x128_amd import workloads as W
from tests.parity import say

pytestmark = pytest.mark.gpu

M, N, K = 384, 512, 1024          # tokens, output channels, input channels (GEMM K: 128-multiples)
T, R, G, NE = 256, 512, 8, 384    # tokens, dispatched rows, experts, expert width


def _step(fp8q, x, w, dy, xt, idx, we_q, we_s, offsets):
    qx, sx = fp8q.quantize_act(x)
    qw, sw = fp8q.quantize_weight(w)
    y = fp8q.gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16)
    qdy, sdy = fp8q.quantize_act(dy)
    qdyt, sdyt = fp8q.quantize_act(dy, fp8q.FP8Q_TILE_128x1)
    qxt, sxt = fp8q.requant_transpose(qx, sx)
    dw = fp8q.gemm(qdyt, sdyt, qxt, sxt, bscale=fp8q.FP8Q_BSCALE_ROW, out_dtype=torch.float32)
    wt_q, wt_s = fp8q.transpose_weight(qw, sw)
    dx = fp8q.dgrad(qdy, sdy, wt_q, wt_s)
    qe, se = fp8q.gather_quantize_act(xt, idx)
    ye = fp8q.grouped_gemm(qe, se, we_q, we_s, offsets, out_dtype=torch.bfloat16)
    return [qx, sx, qw, sw, y, qdy, sdy, qdyt, sdyt, qxt, sxt, dw, wt_q, wt_s, dx, qe, se, ye]


def _fill(rng, x, w, dy, xt):
    x.copy_(torch.from_numpy(rng.standard_t(3, (M, K)).astype(np.float32)))
    w.copy_(torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    dy.copy_(torch.from_numpy((rng.standard_normal((M, N)) * 1e-3).astype(np.float32)))
    xt.copy_(torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)))


def test_training_step_graph_replays_match_eager(fp8q):
    say("graph capture of the fprop/backward/MoE step")
    rng = np.random.default_rng(11)
    dev = "cuda"
    x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    dy = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xt = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    d = W.make_dispatch(T, R, G, K, seed=4)
    idx = torch.from_numpy(d.row_index).to(dev)
    offsets = torch.from_numpy(d.offsets).to(dev)
    we = torch.from_numpy((rng.standard_normal((G, NE, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).to(dev)
    qs = [fp8q.quantize_weight(we[g]) for g in range(G)]
    we_q = torch.stack([q for q, _ in qs])
    we_s = torch.stack([s for _, s in qs])
    args = (x, w, dy, xt, idx, we_q, we_s, offsets)

    _fill(rng, x, w, dy, xt)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(fp8q, *args)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(fp8q, *args)
    torch.cuda.synchronize()

    other = torch.randn((2048, 1024), device=dev).to(torch.bfloat16)
    for rep in range(4):
        if rep % 2 == 1:
            _fill(rng, x, w, dy, xt)  # new values in the captured inputs
        # eager library work between replays
        fp8q.quantize_act(other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in outs]
        ref = [t.cpu() for t in _step(fp8q, *args)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"


def test_splitk_graph_replays_match_eager(fp8q):
    """The split-K GEMM under capture, with a caller workspace and with the
    library's own scratch (the entry point for callers that cannot allocate,
    such as code being captured): 512 x 512 x 8192 (4 tiles, 64 chunks: 16
    slices).  Neither clears memory, so the graphs hold kernel nodes only.
    Each replay, with new operand values and eager split-K work on another
    shape in between, must equal the eager call on the same operands bit for
    bit (the slices are added in a fixed order)."""
    say("graph capture of the split-K GEMM (workspace and no-alloc entries)")
    Mg, Ng, Kg = 512, 512, 8192
    dev = "cuda"
    rng = np.random.default_rng(12)
    need = fp8q.fp8q_gemm_splitk_workspace(Mg, Ng, Kg)
    assert need > 0, "shape expected to split"
    ws = torch.empty((need + 256,), dtype=torch.uint8, device=dev)
    base = (ws.data_ptr() + 255) // 256 * 256
    xa = torch.empty((Mg, Kg), dtype=torch.bfloat16, device=dev)
    xb = torch.empty((Ng, Kg), dtype=torch.bfloat16, device=dev)

    def fill():
        xa.copy_(torch.from_numpy(rng.standard_t(3, (Mg, Kg)).astype(np.float32)))
        xb.copy_(torch.from_numpy((rng.standard_normal((Ng, Kg)) * 0.02).astype(np.float32)))

    fill()
    qa, sa = fp8q.quantize_act(xa)
    qb, sb = fp8q.quantize_weight(xb)
    c_ws = torch.empty((Mg, Ng), dtype=torch.float32, device=dev)
    c_na = torch.empty((Mg, Ng), dtype=torch.float32, device=dev)

    def calls(stream):
        common = (qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), qb.data_ptr(), qb.stride(0),
                  sb.data_ptr(), sb.stride(0), fp8q.FP8Q_BSCALE_BLOCK128, Mg, Ng, Kg)
        assert fp8q.fp8q_quantize_act(xa.data_ptr(), fp8q.FP8Q_BF16, Mg, Kg, Kg, fp8q.FP8Q_TILE_1x128,
                                      qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), stream) == 0
        assert fp8q.fp8q_quantize_weight(xb.data_ptr(), fp8q.FP8Q_BF16, Ng, Kg, Kg, qb.data_ptr(), qb.stride(0),
                                         sb.data_ptr(), sb.stride(0), stream) == 0
        assert fp8q.fp8q_gemm_splitk(*common, c_ws.data_ptr(), fp8q.FP8Q_F32, Ng, 0, 0, base, need, stream) == 0
        assert fp8q.fp8q_gemm_splitk_noalloc(*common, c_na.data_ptr(), fp8q.FP8Q_F32, Ng, 0, 0, stream) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)  # warm-up outside the capture (locates the scratch)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    other_a = torch.randn((300, 5120), device=dev).to(torch.bfloat16)
    other_b = (torch.randn((520, 5120), device=dev) * 0.02).to(torch.bfloat16)
    oqa, osa = fp8q.quantize_act(other_a)
    oqb, osb = fp8q.quantize_weight(other_b)
    for rep in range(4):
        if rep % 2 == 1:
            fill()
        # eager split-K work on another shape between replays (same scratch)
        fp8q.gemm(oqa, osa, oqb, osb, out_dtype=torch.float32)
        oc = torch.empty((300, 520), dtype=torch.float32, device=dev)
        assert fp8q.fp8q_gemm_splitk_noalloc(oqa.data_ptr(), oqa.stride(0), osa.data_ptr(), osa.stride(0),
                                             oqb.data_ptr(), oqb.stride(0), osb.data_ptr(), osb.stride(0),
                                             fp8q.FP8Q_BSCALE_BLOCK128, 300, 520, 5120, oc.data_ptr(),
                                             fp8q.FP8Q_F32, 520, 0, 0,
                                             torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_ws, got_na = c_ws.clone(), c_na.clone()
        calls(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(got_ws, c_ws), f"replay {rep}: workspace split-K differs from eager"
        assert torch.equal(got_na, c_na), f"replay {rep}: no-alloc split-K differs from eager"
        assert torch.equal(c_ws, c_na)
