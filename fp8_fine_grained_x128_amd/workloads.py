"""Seeded synthetic inputs for the fine-grained FP8 linear-layer path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic and imports neither the HIP binding nor the CPU oracle, so
both sides can share it.  Every array is produced on the host with numpy's
PCG64 generator (``numpy.random.default_rng(seed)``), rounded once to the
target dtype with torch's round-to-nearest-even conversion, and returned as a
CPU torch tensor.

Workloads (all seeded with 0 by default):

``tiny``     X fp32 [128 x 512] ~ N(0, 1); W fp32 [256 x 512] ~ N(0, 0.02).
``fprop``    X bf16 [4096 x 7168] ~ Student-t(3) with round(0.001 * 7168) = 7
             columns (drawn without replacement) multiplied by 100 before the
             bf16 rounding; W bf16 [7168 x 7168] ~ N(0, 0.02).
``wgrad``    dY bf16 [8192 x 4096] ~ N(0, 1e-3); X bf16 [8192 x 7168] ~ N(0, 1).
``grouped``  64 experts, W_e bf16 [2048 x 7168] ~ N(0, 0.02); 32768 token rows
             bf16 [x 7168] ~ N(0, 1) grouped by expert with Zipf(1.1) counts.
``longk``    A, B fp32 [1024 x 65536] ~ U[0, 1).
``dispatch`` MoE dispatch of 16384 tokens bf16 [x 7168] ~ N(0, 1) to 64 experts
             with the grouped workload's Zipf(1.1) counts (32768 slots, 2 per
             token on average; the largest expert takes 8208): expert e takes
             counts[e] tokens drawn without replacement from the 16384; the
             row index lists them expert by expert.

The second parameter of N(.,.) is the standard deviation.  The same recipes
scale down (``make_*`` take the sizes) for the parity tests.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _to(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def normal(rng: np.random.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _to(a, dtype)


def student_t_with_outliers(rng: np.random.Generator, rows: int, cols: int, dof: float,
                            outlier_frac: float, outlier_mult: float,
                            dtype: torch.dtype, with_columns: bool = False):
    """Student-t values with round(outlier_frac * cols) columns, drawn without
    replacement, multiplied by outlier_mult; with_columns also returns the
    sorted indices of those columns."""
    a = rng.standard_t(dof, size=(rows, cols)).astype(np.float32)
    n_out = int(round(outlier_frac * cols))
    idx = np.zeros(0, np.int64)
    if n_out:
        idx = rng.choice(cols, size=n_out, replace=False)
        a[:, idx] *= np.float32(outlier_mult)
    t = _to(a, dtype)
    return (t, np.sort(idx)) if with_columns else t


def uniform01(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return _to(rng.random(size=shape, dtype=np.float32), dtype)


def zipf_counts(total: int, groups: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Rows per group: p_r proportional to r^-s (r = 1..groups), largest-
    remainder rounding of total * p (ties to the lower rank), ranks dealt to
    groups by a seeded permutation."""
    r = np.arange(1, groups + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    raw = total * p
    base = np.floor(raw).astype(np.int64)
    rem = raw - base
    left = int(total - base.sum())
    order = sorted(range(groups), key=lambda i: (-rem[i], i))
    for i in order[:left]:
        base[i] += 1
    perm = rng.permutation(groups)
    counts = np.empty(groups, np.int64)
    counts[perm] = base  # rank i goes to group perm[i]
    return counts


@dataclass
class Fprop:
    name: str
    x: torch.Tensor  # [M, K]
    w: torch.Tensor  # [N, K]
    outlier_cols: Optional[np.ndarray] = None  # columns of x scaled x100 (Student-t recipe)


@dataclass
class Wgrad:
    name: str
    dy: torch.Tensor  # [T, Cout]
    x: torch.Tensor   # [T, Cin]


@dataclass
class Grouped:
    name: str
    x: torch.Tensor        # [M_total, K], rows grouped by expert
    w: torch.Tensor        # [G, N, K]
    counts: np.ndarray     # int64[G]
    offsets: np.ndarray    # int32[G + 1]


def make_fprop(M: int, N: int, K: int, *, dtype=torch.bfloat16, seed: int = 0,
               x_dist: str = "normal", w_std: float = 0.02, name: str = "fprop") -> Fprop:
    rng = _rng(seed)
    cols = None
    if x_dist == "student_t":
        x, cols = student_t_with_outliers(rng, M, K, 3.0, 0.001, 100.0, dtype, with_columns=True)
    elif x_dist == "uniform":
        x = uniform01(rng, (M, K), dtype)
    else:
        x = normal(rng, (M, K), 1.0, dtype)
    w = uniform01(rng, (N, K), dtype) if x_dist == "uniform" else normal(rng, (N, K), w_std, dtype)
    return Fprop(name, x, w, cols)


def make_wgrad(T: int, Cout: int, Cin: int, *, dtype=torch.bfloat16, seed: int = 0,
               dy_std: float = 1e-3, name: str = "wgrad") -> Wgrad:
    rng = _rng(seed)
    dy = normal(rng, (T, Cout), dy_std, dtype)
    x = normal(rng, (T, Cin), 1.0, dtype)
    return Wgrad(name, dy, x)


def make_grouped(M_total: int, G: int, N: int, K: int, *, dtype=torch.bfloat16, seed: int = 0,
                 zipf_s: float = 1.1, counts=None, name: str = "grouped") -> Grouped:
    rng = _rng(seed)
    if counts is None:
        counts = zipf_counts(M_total, G, zipf_s, rng)
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.sum() == M_total and len(counts) == G
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    x = normal(rng, (M_total, K), 1.0, dtype)
    w = normal(rng, (G, N, K), 0.02, dtype)
    return Grouped(name, x, w, counts, offsets)


@dataclass
class Dispatch:
    name: str
    x: torch.Tensor          # [tokens, K]
    row_index: np.ndarray    # int32[M_total]: source token of each expert slot
    counts: np.ndarray       # int64[G]
    offsets: np.ndarray      # int32[G + 1]


def make_dispatch(tokens: int, M_total: int, G: int, K: int, *, dtype=torch.bfloat16, seed: int = 0,
                  zipf_s: float = 1.1, name: str = "dispatch") -> Dispatch:
    rng = _rng(seed)
    counts = zipf_counts(M_total, G, zipf_s, rng)
    assert counts.max() <= tokens, "an expert cannot take a token twice"
    idx = np.concatenate([rng.choice(tokens, int(c), replace=False) for c in counts]).astype(np.int32)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    x = normal(rng, (tokens, K), 1.0, dtype)
    return Dispatch(name, x, idx, counts.astype(np.int64), offsets)


# ----------------------------------------------------------------- full sizes

def tiny(seed: int = 0) -> Fprop:
    rng = _rng(seed)
    x = normal(rng, (128, 512), 1.0, torch.float32)
    w = normal(rng, (256, 512), 0.02, torch.float32)
    return Fprop("tiny", x, w)


def fprop(seed: int = 0) -> Fprop:
    return make_fprop(4096, 7168, 7168, x_dist="student_t", seed=seed, name="fprop")


def wgrad(seed: int = 0) -> Wgrad:
    return make_wgrad(8192, 4096, 7168, seed=seed, name="wgrad")


def grouped(seed: int = 0) -> Grouped:
    return make_grouped(32768, 64, 2048, 7168, seed=seed, name="grouped")


def longk(seed: int = 0) -> Fprop:
    return make_fprop(1024, 1024, 65536, dtype=torch.float32, x_dist="uniform", seed=seed,
                      name="longk")


def dispatch(seed: int = 0) -> Dispatch:
    return make_dispatch(16384, 32768, 64, 7168, seed=seed, name="dispatch")


WORKLOADS = {"tiny": tiny, "fprop": fprop, "wgrad": wgrad, "grouped": grouped, "longk": longk,
             "dispatch": dispatch}


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K


def quant_bytes(elements: int, in_bytes: int, tiles: int) -> int:
    """Algorithmic HBM bytes of a quantizer: read inputs, write codes + scales."""
    return elements * (in_bytes + 1) + 4 * tiles


def requant_bytes(elements: int, tiles_in: int, tiles_out: int) -> int:
    """Read codes + 1x128 scales, write codes + 128x1 scales."""
    return 2 * elements + 4 * (tiles_in + tiles_out)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

