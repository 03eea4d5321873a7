"""Shared helpers of the GPU parity tests: move data between torch and the
oracle's numpy layouts, and compare results to the stated bars.

Quantized codes and scales must match bit for bit; GEMM outputs must satisfy
  |C_gpu - C| <= 1e-5 * T        (fp32 output)
  |C_gpu - C| <= 1e-5 * T + 1/2 ulp_bf16(|C| + 1e-5 * T)   (bf16 output)
with C, T = sum_k |a_k b_k| s_a s_b from the FP64 oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

REL_TOL = 1e-5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 copy (bf16 widens exactly) as a contiguous numpy array."""
    return t.detach().to("cpu").float().contiguous().numpy()


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy()


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def dev_codes(q: np.ndarray, device="cuda") -> torch.Tensor:
    """uint8 matrix on the device with a 16-byte-multiple row stride."""
    rows, cols = q.shape
    ld = (cols + 15) // 16 * 16
    buf = torch.zeros((rows, max(ld, 16)), dtype=torch.uint8, device=device)
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(q)).to(device)
    return buf[:, :cols]


def assert_codes_equal(got: np.ndarray, exp: np.ndarray, what: str):
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, (f"{what}: {len(bad)} code mismatches, first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]:#04x} oracle {exp[tuple(bad[0])]:#04x}")


def assert_scales_equal(got: np.ndarray, exp: np.ndarray, what: str):
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    g = np.ascontiguousarray(got, np.float32).view(np.uint32)
    e = np.ascontiguousarray(exp, np.float32).view(np.uint32)
    bad = np.argwhere(g != e)
    assert bad.size == 0, (f"{what}: {len(bad)} scale mismatches, first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]!r} oracle {exp[tuple(bad[0])]!r}")


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.exp2(e - 8)  # ulp = 2^(e-7), half = 2^(e-8)


def gemm_bound(c_ref: np.ndarray, t_ref: np.ndarray, out_dtype) -> np.ndarray:
    b = REL_TOL * t_ref
    if out_dtype == torch.bfloat16:
        b = b + bf16_half_ulp(np.abs(c_ref) + b)
    return b


def assert_gemm_close(got: np.ndarray, c_ref: np.ndarray, t_ref: np.ndarray, out_dtype, what: str):
    got = got.astype(np.float64)
    err = np.abs(got - c_ref)
    bound = gemm_bound(c_ref, t_ref, out_dtype)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0))
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), (f"{what}: {int((err > bound).sum())} outputs out of tolerance; worst at "
                                  f"{worst}: gpu {got[worst]!r} oracle {c_ref[worst]!r} T {t_ref[worst]!r}")
    return float(ratio.max()) if ratio.size else 0.0
