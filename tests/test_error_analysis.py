"""The error statistics that bench.py reports for the method variants (CPU):
the magnitude / direction split is exact, and closed-form cases give their
known values."""
import math
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_split_is_exact_and_closed_forms():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(4000, 128, generator=g, dtype=torch.float64)
    # pure scaling: all of the error is magnitude error
    r = bench.error_analysis(x, 1.5 * x)
    assert all(abs(v - 1.0) < 1e-12 for v in r["magnitude_share"].values())
    assert abs(r["token_scale_abs_log2"]["mean"] - math.log2(1.5)) < 1e-12
    assert abs(r["rel_mse"] - 0.25) < 1e-12
    # a rotation of every row: norms kept, all of the error is direction error
    q, _ = torch.linalg.qr(torch.randn(128, 128, generator=g, dtype=torch.float64))
    r = bench.error_analysis(x, x @ q)
    assert all(abs(v) < 1e-12 for v in r["magnitude_share"].values())
    assert r["token_scale_abs_log2"]["mean"] < 1e-12
    # a mixed error: the split sums to the total per token (checked through a
    # single-token call) and the shares lie in [0, 1]
    xd = x * (1 + 0.1 * torch.randn(4000, 1, generator=g, dtype=torch.float64)) + 0.05 * torch.randn(
        4000, 128, generator=g, dtype=torch.float64)
    r = bench.error_analysis(x, xd)
    assert all(0.0 <= v <= 1.0 for v in r["magnitude_share"].values())
    one = bench.error_analysis(x[:1], xd[:1])
    nk, nd = x[0].norm(), xd[0].norm()
    e_t = float(((x[0] - xd[0]) ** 2).sum())
    e_d = float(2 * nk * nd * (1 - torch.dot(x[0], xd[0]) / (nk * nd)))
    assert abs(one["magnitude_share"]["top_50pct"] * e_t + e_d - e_t) < 1e-9 * e_t


def test_entry_share_of_the_largest_errors():
    x = torch.zeros(100, 128, dtype=torch.float64)
    xd = x.clone()
    xd[0, :] = 1.0                       # 128 of 12800 entries (1 %) hold all of the error
    r = bench.error_analysis(x + 1.0, xd + 1.0)
    assert abs(r["top5pct_entries_share_of_sq_error"] - 1.0) < 1e-12
