"""The seeded generators are deterministic and carry the planted structure."""
import numpy as np
import torch

from precision_quantization_row_amd import workloads


def test_deterministic():
    a = workloads.make("tiny_rowscale")
    b = workloads.make("tiny_rowscale")
    assert torch.equal(a.x.view(torch.int16), b.x.view(torch.int16))
    assert a.x.dtype == torch.bfloat16 and a.shape == (256, 256)


def test_outliers_fraction():
    w = workloads.make("outliers", (512, 512))
    big = (w.x.float().abs() >= 100).sum().item()
    assert big == w.notes["n_outliers"] == 512 * 512 // 1000


def test_moe_layout():
    w = workloads.make("moe_groups", (2000, 64))
    ge = w.group_end
    assert ge.numel() == 16 and int(w.group_rows.sum()) == 2000
    pad = torch.diff(torch.cat([torch.zeros(1, dtype=torch.int64), ge]))
    assert bool((pad % 128 == 0).all()) and bool((pad >= w.group_rows).all())
    start = 0
    for g in range(16):
        n = int(w.group_rows[g])
        assert not w.x[start + n:int(ge[g])].float().abs().sum()
        start = int(ge[g])


def test_fp32_edge_structure():
    w = workloads.make("fp32_edge")
    x = w.x.numpy()
    assert x.shape == (4097, 2880) and x.dtype == np.float32
    assert not x[w.notes["zero_row"]].any()
    c, r = w.notes["single_nonzero_col"]
    nz = np.nonzero(x[:, c])[0]
    assert nz.tolist() == [r]
    sub = np.abs(np.delete(x[w.notes["subnormal_row"]], c))  # column c is zeroed
    assert (sub < np.finfo(np.float32).tiny).all() and (sub > 0).all()
    lim = np.finfo(np.float32).max / 448
    er = np.abs(np.delete(x[w.notes["extreme_rows"][0]], c))
    assert (er >= 0.5 * lim * 0.999).all() and (er <= 0.99 * lim * 1.001).all()
    assert np.isfinite(x).all()
