"""GPU parity of the power-of-two-scale GEMM datapaths (FP8Q_GEMM_POW2_SCALES,
alone and with FP8Q_GEMM_MMA_FP8) against the FP64 oracle, on operands the
oracle quantized with power-of-two scales.

Bounds, with T = sum_k |a_k b_k| s_a s_b:
  bf16 fold (POW2 alone): the default bound 1e-5 T (+ half a bf16 ulp);
  block-scaled FP8 (POW2 | MMA_FP8): 2^-10 T on top of it (the FP8
  instruction's in-run truncation, see the accumulation probe tests).
The long-K test reports the error of every datapath on prefixes of a
K = 65536 contraction; with no promotion step the two power-of-two paths
accumulate the whole K in the matrix core, so this is where a limited
accumulator would show growth with K.
"""
import numpy as np
import pytest
import torch

from fp8_fine_grained_x128_amd import workloads as W
from tests.parity import assert_gemm_close, dev, dev_codes, gemm_bound, host_f32, say

pytestmark = pytest.mark.gpu
POW2 = 1
FOLD = 2          # FP8Q_GEMM_POW2_SCALES
SCALED = 2 | 1    # FP8Q_GEMM_POW2_SCALES | FP8Q_GEMM_MMA_FP8
FP8_EXTRA = 2.0 ** -10


def _operands(oracle, M, N, K, mode, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x, POW2)
    if mode == 0:
        qb, sb = oracle.quantize_weight_128x128(w, POW2)
        sb_dev = sb
    else:
        qbt, sbt = oracle.quantize_act_128x1(w.T.copy(), POW2)
        qb, sb, sb_dev = qbt.T.copy(), sbt.T.copy(), sbt
    return qa, sa, qb, sb, sb_dev


def _check(got, c_ref, t_ref, out_dtype, flags, what):
    if flags == FOLD:
        return assert_gemm_close(got, c_ref, t_ref, out_dtype, what)
    err = np.abs(got.astype(np.float64) - c_ref)
    bound = gemm_bound(c_ref, t_ref, out_dtype) + FP8_EXTRA * t_ref
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} outputs beyond the FP8 bound"
    return float((err / np.where(bound > 0, bound, 1)).max())


CASES = [(300, 520, 640), (256, 256, 128), (1, 1, 128), (513, 130, 1024), (64, 1040, 384)]


@pytest.mark.parametrize("flags", [FOLD, SCALED])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", CASES)
def test_pow2_gemm_parity(fp8q, oracle, flags, mode, out_dtype, shape):
    M, N, K = shape
    say(f"pow2 gemm flags={flags} mode={mode} {out_dtype} {shape}")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, mode, seed=M + 3 * N + K + mode)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, mode)
    out = fp8q.gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev_codes(qb), dev(np.ascontiguousarray(sb_dev)),
                    bscale=mode, out_dtype=out_dtype, flags=flags)
    torch.cuda.synchronize()
    r = _check(host_f32(out), c_ref, t_ref, out_dtype, flags, f"pow2 gemm {shape}")
    say(f"  worst err/bound = {r:.3f}")


@pytest.mark.parametrize("flags", [FOLD, SCALED])
@pytest.mark.parametrize("mode", [0, 1])
def test_pow2_gemm_bitexact(fp8q, oracle, flags, mode):
    """Codes +-2^i (|i| <= 3) and power-of-two scales constant along K for
    each row of A and of B: every product and running sum is exact in fp32
    (products within 12 binary orders of each other, inside the FP8
    instruction's window), so both datapaths must reproduce the oracle bit for
    bit."""
    M, N, K = 300, 300, 512
    rng = np.random.default_rng(20 + mode)
    a = (rng.choice([-1.0, 1.0], (M, K)) * np.exp2(rng.integers(-3, 4, (M, K)))).astype(np.float32)
    b = (rng.choice([-1.0, 1.0], (N, K)) * np.exp2(rng.integers(-3, 4, (N, K)))).astype(np.float32)
    qa = oracle.e4m3_encode(a).reshape(M, K)
    qb = oracle.e4m3_encode(b).reshape(N, K)
    nk = K // 128
    sa = np.repeat(np.exp2(rng.integers(-4, 5, (M, 1))), nk, axis=1).astype(np.float32)
    if mode == 0:
        sb = np.repeat(np.exp2(rng.integers(-4, 5, (-(-N // 128), 1))), nk, axis=1).astype(np.float32)
        sb_dev = sb
    else:
        sb = np.repeat(np.exp2(rng.integers(-4, 5, (N, 1))), nk, axis=1).astype(np.float32)
        sb_dev = np.ascontiguousarray(sb.T)
    c_ref, _ = oracle.gemm(qa, sa, qb, sb, mode)
    out = fp8q.gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev_codes(qb), dev(sb_dev), bscale=mode,
                    out_dtype=torch.float32, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(out).astype(np.float64), c_ref)


@pytest.mark.parametrize("flags", [FOLD, SCALED])
def test_pow2_grouped(fp8q, oracle, flags):
    counts, N, K = [0, 37, 300, 129, 1], 384, 512
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(30)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x, POW2)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g], POW2) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    say(f"pow2 grouped flags={flags}")
    out = fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                            out_dtype=torch.bfloat16, flags=flags)
    torch.cuda.synchronize()
    _check(host_f32(out), c_ref.reshape(M, N), t_ref.reshape(M, N), torch.bfloat16, flags, "pow2 grouped")


def test_longk_all_datapaths(fp8q, oracle):
    """A, B fp32 1024 x 65536 U[0,1) quantized with power-of-two scales; the
    four datapaths on prefixes K' = 128 .. 65536 against the oracle's prefix
    sums.  Reports max and mean err/T per K'; each stays within its bound."""
    wl = W.longk()
    qa, sa = oracle.quantize_act_1x128(host_f32(wl.x), POW2)
    qb, sb = oracle.quantize_weight_128x128(host_f32(wl.w), POW2)
    a_d, sa_d = dev_codes(qa), dev(np.ascontiguousarray(sa.T))
    b_d, sb_d = dev_codes(qb), dev(sb)
    rng = np.random.default_rng(4)
    im = rng.integers(0, 1024, 4096).astype(np.int64)
    jn = rng.integers(0, 1024, 4096).astype(np.int64)
    names = {0: "default", 1: "fp8", FOLD: "bf16-fold", SCALED: "fp8-scaled"}
    for Kp in [128 * 2 ** j for j in range(10)]:
        c, t = oracle.gemm_entries(qa, sa, qb, sb, im, jn, 0, K=Kp)
        line = []
        for flags in (0, 1, FOLD, SCALED):
            out = torch.empty((1024, 1024), dtype=torch.float32, device="cuda")
            rc = fp8q.binding.fp8q_gemm_ex(a_d.data_ptr(), a_d.stride(0), sa_d.data_ptr(), sa_d.stride(0),
                                           b_d.data_ptr(), b_d.stride(0), sb_d.data_ptr(), sb_d.stride(0), 0,
                                           1024, 1024, Kp, out.data_ptr(), 0, 1024, 0, flags,
                                           torch.cuda.current_stream().cuda_stream)
            assert rc == 0
            torch.cuda.synchronize()
            got = host_f32(out)[im, jn].astype(np.float64)
            rel = np.abs(got - c) / t
            line.append(f"{names[flags]} {rel.max():.2e}/{rel.mean():.2e}")
            bound = 1e-5 + (FP8_EXTRA if flags & 1 else 0.0)
            assert np.all(rel <= bound), (names[flags], Kp, rel.max())
        say(f"  K'={Kp}: " + "; ".join(line))


@pytest.mark.parametrize("flags", [1, FOLD, SCALED])
@pytest.mark.parametrize("mode", [0, 1])
def test_strip_layout_all_datapaths(fp8q, oracle, flags, mode):
    """M = 4096 selects the 256x448 strip layout; N = 7000 leaves a ragged last
    strip.  The 192-wide second tile takes one B scale per 16-column subtile
    in every datapath.  Operands use power-of-two scales (valid for all
    three flags); sampled outputs against the oracle."""
    M, N, K = 4096, 7000, 256
    say(f"strip layout flags={flags} mode={mode}")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, mode, seed=5 + flags + mode)
    out = fp8q.gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev_codes(qb),
                    dev(np.ascontiguousarray(sb_dev)), bscale=mode, out_dtype=torch.float32, flags=flags)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    im = np.concatenate([np.repeat([0, 255, 4095], N), rng.integers(0, M, 3000)]).astype(np.int64)
    jn = np.concatenate([np.tile(np.arange(N), 3), rng.integers(0, N, 3000)]).astype(np.int64)
    c, t = oracle.gemm_entries(qa, sa, qb, sb, im, jn, mode)
    got = host_f32(out)[im, jn]
    if flags == FOLD:
        assert_gemm_close(got, c, t, torch.float32, "strip fold")
    else:
        err = np.abs(got.astype(np.float64) - c)
        assert np.all(err <= (1e-5 + FP8_EXTRA) * t), f"flags={flags}: {int((err > (1e-5 + FP8_EXTRA) * t).sum())} out"
