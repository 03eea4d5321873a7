"""GPU parity of the quantizers against the CPU oracle: codes and scales
bit-exact, on ragged shapes spanning several tiles, on edge values, and
exhaustively for the E4M3 conversion of every fp32 value of magnitude <= 448."""
import numpy as np
import pytest
import torch

from tests.parity import (assert_codes_equal, assert_scales_equal, dev, dev_codes, host_f32, host_u8,
                          say)

pytestmark = pytest.mark.gpu


def _padded(x: torch.Tensor, align_elems: int) -> torch.Tensor:
    """Copy of x on the GPU inside a buffer whose row stride is a multiple of
    align_elems (so the tensor is a strided view, ld > cols)."""
    rows, cols = x.shape
    ld = (cols + align_elems - 1) // align_elems * align_elems + align_elems
    buf = torch.zeros((rows, ld), dtype=x.dtype, device="cuda")
    buf[:, :cols] = x.to("cuda")
    return buf[:, :cols]


def _inputs(rows, cols, dtype, seed, kind="t"):
    rng = np.random.default_rng(seed)
    if kind == "t":
        a = rng.standard_t(3, (rows, cols)).astype(np.float32)
        a[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= 100
    elif kind == "wide":
        e = rng.integers(-130, 20, size=(rows, cols))
        a = (rng.choice([-1.0, 1.0], (rows, cols)) * rng.random((rows, cols)) * np.exp2(e)).astype(np.float32)
    else:
        a = rng.standard_normal((rows, cols)).astype(np.float32)
    t = torch.from_numpy(a).to(dtype)
    # edge rows: zeros, signed zeros, subnormal-scale data, exact 448 multiples
    if rows > 4:
        t[0, :] = 0
        t[1, :] = -0.0
        t[2, :] = torch.from_numpy((rng.standard_normal(cols) * 1e-38).astype(np.float32)).to(dtype)
        t[3, : min(cols, 5)] = torch.tensor([448.0, -448.0, 1.0, -0.0, 3.5], dtype=dtype)[: min(cols, 5)]
    return t


SHAPES = [(1, 128), (5, 7), (300, 1000), (257, 1032), (64, 7168), (130, 200)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_act_1x128(fp8q, oracle, dtype, shape):
    rows, cols = shape
    say(f"quantize_act 1x128 {dtype} {shape}")
    x = _inputs(rows, cols, dtype, seed=rows * 31 + cols)
    xd = _padded(x, 8 if dtype == torch.bfloat16 else 4)
    q, s = fp8q.quantize_act(xd, fp8q.FP8Q_TILE_1x128)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_1x128(host_f32(x))
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so.T, "scales")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 200), (1000, 257), (128, 128), (7, 5), (129, 4096)])
def test_quantize_act_128x1(fp8q, oracle, dtype, shape):
    rows, cols = shape
    say(f"quantize_act 128x1 {dtype} {shape}")
    x = _inputs(rows, cols, dtype, seed=rows * 17 + cols, kind="n")
    xd = _padded(x, 8 if dtype == torch.bfloat16 else 4)
    q, s = fp8q.quantize_act(xd, fp8q.FP8Q_TILE_128x1)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_128x1(host_f32(x))
    assert_codes_equal(host_u8(q), qo.T, "codes (transposed)")
    assert_scales_equal(host_f32(s), so, "scales")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(300, 1000), (256, 7168), (129, 131), (1, 16)])
def test_quantize_weight(fp8q, oracle, dtype, shape):
    N, K = shape
    say(f"quantize_weight {dtype} {shape}")
    w = _inputs(N, K, dtype, seed=N + 7 * K, kind="wide" if N == 129 else "n")
    wd = _padded(w, 8 if dtype == torch.bfloat16 else 4)
    q, s = fp8q.quantize_weight(wd)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_weight_128x128(host_f32(w))
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so, "scales")


@pytest.mark.parametrize("shape", [(300, 1000), (1000, 300), (256, 256), (8, 200), (129, 1040)])
def test_requant_transpose(fp8q, oracle, shape):
    """Input codes/scales come from the oracle's own 1x128 quantization."""
    rows, cols = shape
    say(f"requant_transpose {shape}")
    x = host_f32(_inputs(rows, cols, torch.bfloat16, seed=rows + cols))
    q1, s1 = oracle.quantize_act_1x128(x)
    q2, s2 = oracle.requant_1x128_to_128x1(q1, s1)
    qt, st = fp8q.requant_transpose(dev_codes(q1), dev(np.ascontiguousarray(s1.T)))
    torch.cuda.synchronize()
    assert_codes_equal(host_u8(qt), q2.T, "codes (transposed)")
    assert_scales_equal(host_f32(st), s2, "scales")


def test_chain_quantize_then_requant(fp8q, oracle):
    rows, cols = 384, 640
    say("chain quantize_act -> requant_transpose")
    x = _inputs(rows, cols, torch.bfloat16, seed=99)
    q, s = fp8q.quantize_act(x.cuda())
    qt, st = fp8q.requant_transpose(q, s)
    torch.cuda.synchronize()
    q1, s1 = oracle.quantize_act_1x128(host_f32(x))
    q2, s2 = oracle.requant_1x128_to_128x1(q1, s1)
    assert_codes_equal(host_u8(qt), q2.T, "codes")
    assert_scales_equal(host_f32(st), s2, "scales")


@pytest.mark.parametrize("sign", [0, 1])
def test_e4m3_conversion_exhaustive(fp8q, oracle, sign):
    """Every fp32 value with |y| <= 448 goes through the quantizer's convert
    path: tiles [448, y_1 .. y_127] have s = 1 exactly, so the codes are
    e4m3(y_i) and must equal the oracle's encoder on the same patterns."""
    per_row = 127
    rows_per_chunk = 1 << 21
    last = 0x43E00000  # 448.0
    total = last + 1
    done = 0
    say(f"exhaustive conversion sign={sign}")
    while done < total:
        n = min(per_row * rows_per_chunk, total - done)
        rows = -(-n // per_row)
        pats = torch.arange(done, done + rows * per_row, dtype=torch.int64, device="cuda")
        pats = torch.clamp(pats, max=last)  # pad the tail with the last pattern
        if sign:
            pats = pats + 0x80000000
        pats = torch.where(pats >= 2 ** 31, pats - 2 ** 32, pats).to(torch.int32)
        vals = pats.view(torch.float32).reshape(rows, per_row)
        x = torch.empty((rows, 128), dtype=torch.float32, device="cuda")
        x[:, 0] = 448.0
        x[:, 1:] = vals
        q, s = fp8q.quantize_act(x)
        torch.cuda.synchronize()
        assert torch.all(s == 1.0).item()
        got = host_u8(q[:, 1:]).reshape(-1)[:n]
        exp = oracle.e4m3_encode_patterns((0x80000000 if sign else 0) + done, n)
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, f"pattern {done + int(bad[0]):#x}: gpu {got[bad[0]]:#x} oracle {exp[bad[0]]:#x}"
        done += n


def test_quantize_act_1x128_many_row_groups(fp8q, oracle):
    """More 16-row groups than one grid dimension holds (65535): the row
    groups continue in the third grid dimension.  bf16, ragged columns."""
    rows, cols = 65535 * 16 + 37, 200
    say(f"quantize_act 1x128 bf16 {rows}x{cols} (row groups past 65535)")
    rng = np.random.default_rng(77)
    x = torch.from_numpy(rng.standard_normal((rows, cols), dtype=np.float32)).to(torch.bfloat16)
    q, s = fp8q.quantize_act(_padded(x, 8))
    torch.cuda.synchronize()
    qo, so = oracle.quantize_act_1x128(host_f32(x))
    assert_codes_equal(host_u8(q), qo, "codes")
    assert_scales_equal(host_f32(s), so.T, "scales")


@pytest.mark.parametrize("tile", ["1x128", "128x1", "128x128"])
def test_nonfinite_inputs_stay_in_their_tile(fp8q, oracle, tile):
    """Non-finite inputs are outside the quantizers' contract (their tile's
    codes and scale are unspecified), but the call completes and every other
    tile is exactly what the oracle gives."""
    rows, cols = 300, 520
    say(f"non-finite inputs, {tile}")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    bad = [(5, 3, np.inf), (140, 200, np.nan), (299, 519, -np.inf)]
    for r, c, v in bad:
        x[r, c] = v
    clean = x.copy()
    for r, c, _ in bad:
        clean[r, c] = 0.0
    xd = torch.from_numpy(x).cuda()
    if tile == "1x128":
        q, s = fp8q.quantize_act(xd)
        qo, so = oracle.quantize_act_1x128(clean)
        got_q, got_s, exp_s = host_u8(q), host_f32(s).T, so
        tiles = [(r, c // 128) for r, c, _ in bad]
        qmask = np.ones(qo.shape, bool)
        smask = np.ones(so.shape, bool)
        for r, cb in tiles:
            qmask[r, 128 * cb:128 * cb + 128] = False
            smask[r, cb] = False
    elif tile == "128x1":
        q, s = fp8q.quantize_act(xd, fp8q.FP8Q_TILE_128x1)
        qo, so = oracle.quantize_act_128x1(clean)
        got_q, got_s, exp_s = host_u8(q).T, host_f32(s), so
        qmask = np.ones(qo.shape, bool)
        smask = np.ones(so.shape, bool)
        for r, c, _ in bad:
            qmask[128 * (r // 128):128 * (r // 128) + 128, c] = False
            smask[r // 128, c] = False
    else:
        q, s = fp8q.quantize_weight(xd)
        qo, so = oracle.quantize_weight_128x128(clean)
        got_q, got_s, exp_s = host_u8(q), host_f32(s), so
        qmask = np.ones(qo.shape, bool)
        smask = np.ones(so.shape, bool)
        for r, c, _ in bad:
            rb, cb = r // 128, c // 128
            qmask[128 * rb:128 * rb + 128, 128 * cb:128 * cb + 128] = False
            smask[rb, cb] = False
    torch.cuda.synchronize()
    assert_codes_equal(got_q[qmask], qo[qmask], "codes outside the non-finite tiles")
    assert_scales_equal(got_s[smask], exp_s[smask], "scales outside the non-finite tiles")
