"""The seeded input generators are reproducible and follow their recipes."""
import numpy as np
import torch

from fp8_fine_grained_x128_amd import workloads as W


def test_zipf_counts():
    c = W.zipf_counts(32768, 64, 1.1, np.random.default_rng(0))
    assert c.sum() == 32768 and c.max() == 8208 and c.min() == 85
    assert (c < 128).sum() == 20
    top = sorted(c, reverse=True)[:4]
    assert top == [8208, 3829, 2451, 1786]


def test_reproducible_small():
    a = W.make_fprop(64, 256, 512, x_dist="student_t", seed=0)
    b = W.make_fprop(64, 256, 512, x_dist="student_t", seed=0)
    assert torch.equal(a.x, b.x) and torch.equal(a.w, b.w)
    assert a.x.dtype == torch.bfloat16
    c = W.make_fprop(64, 256, 512, x_dist="student_t", seed=1)
    assert not torch.equal(a.x, c.x)


def test_outlier_columns():
    f = W.make_fprop(512, 128, 7168, x_dist="student_t", seed=0)
    col_amax = f.x.float().abs().amax(dim=0)
    big = torch.topk(col_amax, 7).values.min()
    rest = torch.sort(col_amax, descending=True).values[7:].max()
    assert big > 10 * rest / 3  # the seven x100 columns stand out


def test_tiny_and_grouped_shapes():
    t = W.tiny()
    assert t.x.shape == (128, 512) and t.w.shape == (256, 512) and t.x.dtype == torch.float32
    g = W.make_grouped(1000, 8, 256, 256, seed=0)
    assert g.offsets[0] == 0 and g.offsets[-1] == 1000 and g.w.shape == (8, 256, 256)
    assert np.all(np.diff(g.offsets) == g.counts)
