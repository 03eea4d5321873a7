"""GPU parity of the block-scaled GEMMs against the FP64 oracle.

Operands are quantized by the oracle (never by the HIP path) and uploaded;
the GPU output must satisfy the tolerance of tests/parity.py everywhere.
Power-of-two inputs with integer products give exactly representable sums,
where the GPU must match the oracle bit for bit."""
import numpy as np
import pytest
import torch

from tests.parity import assert_gemm_close, dev, dev_codes, host_f32, say

pytestmark = pytest.mark.gpu


def _operands(oracle, M, N, K, mode, seed, x_kind="t"):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (M, K)).astype(np.float32) if x_kind == "t" else rng.random((M, K), np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)          # sa [M][K/128]
    if mode == 0:
        qb, sb = oracle.quantize_weight_128x128(w)  # sb [N/128][K/128]
        sb_dev = sb
    else:
        qb, sbt = oracle.quantize_act_128x1(w.T.copy())  # per-row (of B) per 128-K scales
        qb = qb.T.copy()                                  # [N][K]
        sb = sbt.T.copy()                                 # oracle layout [N][K/128]
        sb_dev = sbt                                      # device layout [K/128][N]
    return qa, sa, qb, sb, sb_dev


def _run(fp8q, qa, sa, qb, sb_dev, mode, out_dtype, c=None, accumulate=False):
    a = dev_codes(qa)
    b = dev_codes(qb)
    sa_d = dev(np.ascontiguousarray(sa.T))
    sb_d = dev(np.ascontiguousarray(sb_dev))
    out = fp8q.gemm(a, sa_d, b, sb_d, bscale=mode, out_dtype=out_dtype, c=c, accumulate=accumulate)
    torch.cuda.synchronize()
    return out


CASES = [
    (300, 520, 640),   # ragged M and N across several 256-tiles, 5 chunks
    (256, 256, 128),   # one tile, one chunk
    (1, 1, 128),       # degenerate
    (513, 130, 1024),  # ragged both ways, 8 chunks
    (64, 1040, 384),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", CASES)
def test_gemm_parity(fp8q, oracle, mode, out_dtype, shape):
    M, N, K = shape
    say(f"gemm mode={mode} {out_dtype} {shape}")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, mode, seed=M + N + K + mode)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, mode)
    out = _run(fp8q, qa, sa, qb, sb_dev, mode, out_dtype)
    r = assert_gemm_close(host_f32(out), c_ref, t_ref, out_dtype, f"gemm {shape}")
    say(f"  worst err/bound = {r:.3f}")


def test_gemm_accumulate(fp8q, oracle):
    M, N, K = 300, 520, 640
    say("gemm accumulate")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, 0, seed=5)
    c_ref, t_ref = oracle.gemm(qa, sa, qb, sb, 0)
    base = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    c = dev(base)
    _run(fp8q, qa, sa, qb, sb_dev, 0, torch.float32, c=c, accumulate=True)
    # base + C: the fp32 addition adds at most half an fp32 ulp of the sum
    got = host_f32(c).astype(np.float64)
    exp = base.astype(np.float64) + c_ref
    bound = 1e-5 * t_ref + np.abs(exp) * 2.0 ** -24 + 1e-30
    assert np.all(np.abs(got - exp) <= bound)


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_power_of_two_bitexact(fp8q, oracle, mode):
    """Codes of +-2^i (|i| <= 3) and power-of-two scales that are constant
    along K for each row of A and of B: every product, chunk partial and
    running total is an exact fp32 value (at most 21 significant bits), so the
    GPU must reproduce the oracle bit for bit."""
    M, N, K = 300, 300, 512
    say(f"gemm pow2 exact mode={mode}")
    rng = np.random.default_rng(2 + mode)
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
    out = _run(fp8q, qa, sa, qb, sb_dev, mode, torch.float32)
    assert np.array_equal(host_f32(out).astype(np.float64), c_ref)


def test_gemm_scale_doubling_and_determinism(fp8q, oracle):
    M, N, K = 300, 520, 640
    say("gemm invariants")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, 0, seed=7)
    c1 = host_f32(_run(fp8q, qa, sa, qb, sb_dev, 0, torch.float32))
    c2 = host_f32(_run(fp8q, qa, sa, qb, sb_dev, 0, torch.float32))
    assert np.array_equal(c1, c2)  # deterministic
    c3 = host_f32(_run(fp8q, qa, sa * np.float32(2), qb, sb_dev, 0, torch.float32))
    assert np.array_equal(c3, 2 * c1)  # power-of-two scaling is exact
    perm = np.random.default_rng(0).permutation(M)
    c4 = host_f32(_run(fp8q, qa[perm], sa[perm], qb, sb_dev, 0, torch.float32))
    assert np.array_equal(c4, c1[perm])  # rows are independent


GROUPED = [
    ([0, 37, 300, 129, 1, 0], 384, 512),
    ([256, 0, 0, 511], 256, 256),
    ([5], 130, 128),
]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", GROUPED)
def test_grouped_gemm_parity(fp8q, oracle, case, out_dtype):
    counts, N, K = case
    G = len(counts)
    say(f"grouped counts={counts} N={N} K={K} {out_dtype}")
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(G + N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    a = dev_codes(qa)
    b = dev(qb)  # [G][N][K], K multiple of 128 -> 16-byte rows
    out = fp8q.grouped_gemm(a, dev(np.ascontiguousarray(sa.T)), b, dev(sb), dev(off), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert_gemm_close(host_f32(out), c_ref.reshape(M, N), t_ref.reshape(M, N), out_dtype, "grouped")
    # grouped == per-expert plain GEMM (same tile path)
    for g in range(G):
        if counts[g] == 0:
            continue
        rows = slice(off[g], off[g + 1])
        single = fp8q.gemm(dev_codes(qa[rows]), dev(np.ascontiguousarray(sa[rows].T)), dev_codes(qb[g]),
                           dev(sb[g]), out_dtype=out_dtype, split_k=False)
        torch.cuda.synchronize()
        assert torch.equal(single.cpu(), out[rows].cpu())


def test_grouped_many_groups_multiple_rounds(fp8q, oracle):
    """150 experts with seeded counts in [0, 300] plus forced boundary sizes
    (0, 1, 127, 128, 129, 255, 256, 257, 384, 385): the tile list holds 344
    tiles, more than one round of the persistent grid, with every full-height
    tile ordered before every 128-row remainder tile.  Checked against the
    oracle on all outputs and bit for bit against per-expert plain GEMMs."""
    rng = np.random.default_rng(150)
    counts = list(rng.integers(0, 301, 140)) + [0, 1, 127, 128, 129, 255, 256, 257, 384, 385]
    counts = [int(c) for c in rng.permutation(np.array(counts))]
    G, N, K = len(counts), 512, 128
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    say(f"grouped G={G} M={M} N={N} K={K}")
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    out = fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host_f32(out), c_ref.reshape(M, N), t_ref.reshape(M, N), torch.float32, "grouped G=150")
    for g in range(G):
        if counts[g] == 0:
            continue
        rows = slice(off[g], off[g + 1])
        single = fp8q.gemm(dev_codes(qa[rows]), dev(np.ascontiguousarray(sa[rows].T)), dev_codes(qb[g]),
                           dev(sb[g]), out_dtype=torch.float32, split_k=False)
        torch.cuda.synchronize()
        assert torch.equal(single.cpu(), out[rows].cpu()), g


def _grouped_operands(oracle, M, G, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    return qa, sa, np.stack(qbs), np.stack(sbs)


def test_grouped_tile_height_classes(fp8q, oracle):
    """An expert's last row tile runs 64, 128, 192 or 256 rows high; expert
    sizes on both sides of every class boundary (and of whole 256-row tiles),
    all outputs against the oracle and bit for bit against per-expert plain
    GEMMs."""
    counts = [1, 64, 65, 128, 129, 192, 193, 256, 257, 320, 321, 384, 385, 448, 449, 512, 0, 63]
    G, N, K = len(counts), 384, 256
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    say(f"grouped tile classes G={G} M={M}")
    qa, sa, qb, sb = _grouped_operands(oracle, M, G, N, K, 7)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    for out_dtype in (torch.float32, torch.bfloat16):
        out = fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                                out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert_gemm_close(host_f32(out), c_ref.reshape(M, N), t_ref.reshape(M, N), out_dtype, "tile classes")
        for g in range(G):
            if counts[g] == 0:
                continue
            rows = slice(off[g], off[g + 1])
            single = fp8q.gemm(dev_codes(qa[rows]), dev(np.ascontiguousarray(sa[rows].T)), dev_codes(qb[g]),
                               dev(sb[g]), out_dtype=out_dtype, split_k=False)
            torch.cuda.synchronize()
            assert torch.equal(single.cpu(), out[rows].cpu()), g


@pytest.mark.parametrize("raw", [[0, 100, 250, 400, 500],    # past M_total
                                 [0, 200, 150, 300, 300],    # decreasing
                                 [-50, 100, 200, 300, 290]])  # negative, then decreasing at the end
def test_grouped_offsets_out_of_range(fp8q, oracle, raw):
    """Offsets from a faulty routing step: the kernel clamps them to
    [0, M_total] and makes them non-decreasing (off'[0] = clamp(off[0]),
    off'[g+1] = clamp(off[g+1], off'[g], M_total)), so no tile reads past A or
    its scales and no row outside [off'[0], off'[G]) of C, nor any row past
    C, is written.  C sits in a larger buffer whose guard rows must survive."""
    G, N, K, M = 4, 256, 256, 300
    qa, sa, qb, sb = _grouped_operands(oracle, M, G, N, K, 8)
    clamped = [min(max(raw[0], 0), M)]
    for v in raw[1:]:
        clamped.append(min(max(v, clamped[-1]), M))
    clamped = np.array(clamped, np.int32)
    say(f"grouped offsets {raw} -> {list(clamped)}")
    buf = torch.full((M + 64, N), -7.0, dtype=torch.float32, device="cuda")
    c = buf[:M]
    fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb),
                      dev(np.array(raw, np.int32)), c=c)
    torch.cuda.synchronize()
    got = host_f32(buf)
    assert np.all(got[M:] == -7.0), "rows past C were written"
    lo, hi = int(clamped[0]), int(clamped[-1])
    assert np.all(got[:lo] == -7.0) and np.all(got[hi:M] == -7.0)
    if hi > lo:
        mm, nn = np.meshgrid(np.arange(lo, hi), np.arange(N), indexing="ij")
        c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, clamped, mm.ravel(), nn.ravel())
        assert_gemm_close(got[lo:hi], c_ref.reshape(hi - lo, N), t_ref.reshape(hi - lo, N), torch.float32,
                          "clamped offsets")


def test_grouped_max_groups(fp8q, oracle):
    """1024 experts (the largest accepted count), almost all empty: the tile
    tables fill their whole LDS space and the search must skip runs of empty
    groups, including at both ends."""
    G, N, K = 1024, 256, 128
    counts = np.zeros(G, np.int64)
    for g, c in [(1, 3), (7, 300), (500, 128), (501, 129), (1022, 40)]:
        counts[g] = c
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    say(f"grouped G={G} M={M}")
    rng = np.random.default_rng(1024)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_act_1x128(x)
    qbs, sbs = zip(*[oracle.quantize_weight_128x128(w[g]) for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c_ref, t_ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mm.ravel(), nn.ravel())
    out = fp8q.grouped_gemm(dev_codes(qa), dev(np.ascontiguousarray(sa.T)), dev(qb), dev(sb), dev(off),
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(host_f32(out), c_ref.reshape(M, N), t_ref.reshape(M, N), torch.float32, "grouped G=1024")


@pytest.mark.parametrize("N", [7000, 6936])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_strip_layout_ragged(fp8q, oracle, N, mode):
    """M = 4096 rows make the library cut N into 448-wide strips (a 256x256
    then a 256x192 tile per work-group).  N = 7000 leaves a last strip whose
    second tile has 24 columns; N = 6936 one whose second tile starts past
    N.  Every column of a few rows at tile edges and random entries are
    checked against the oracle."""
    M, K = 4096, 384
    say(f"gemm strip layout N={N} mode={mode}")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, mode, seed=N + mode)
    out = _run(fp8q, qa, sa, qb, sb_dev, mode, torch.float32)
    rng = np.random.default_rng(9)
    rows = [0, 255, 256, 2047, 4095]
    im = np.concatenate([np.repeat(rows, N), rng.integers(0, M, 4000)]).astype(np.int64)
    jn = np.concatenate([np.tile(np.arange(N), len(rows)), rng.integers(0, N, 4000)]).astype(np.int64)
    c, t = oracle.gemm_entries(qa, sa, qb, sb, im, jn, mode)
    assert_gemm_close(host_f32(out)[im, jn], c, t, torch.float32, f"strip N={N}")


def test_gemm_strip_layout_accumulate(fp8q, oracle):
    """Strip layout with fp32 output added to an existing C."""
    M, N, K = 4096, 7000, 256
    say("gemm strip layout accumulate")
    qa, sa, qb, sb, sb_dev = _operands(oracle, M, N, K, 0, seed=77)
    base = np.random.default_rng(3).standard_normal((M, N)).astype(np.float32)
    c = dev(base)
    _run(fp8q, qa, sa, qb, sb_dev, 0, torch.float32, c=c, accumulate=True)
    rng = np.random.default_rng(4)
    im = np.concatenate([np.repeat([0, 2047, 4095], N), rng.integers(0, M, 3000)]).astype(np.int64)
    jn = np.concatenate([np.tile(np.arange(N), 3), rng.integers(0, N, 3000)]).astype(np.int64)
    cr, tr = oracle.gemm_entries(qa, sa, qb, sb, im, jn, 0)
    got = host_f32(c)[im, jn].astype(np.float64)
    exp = base[im, jn].astype(np.float64) + cr
    assert np.all(np.abs(got - exp) <= 1e-5 * tr + np.abs(exp) * 2.0 ** -24 + 1e-30)
