"""The error statistics that bench.py reports for the method variants (CPU):
the magnitude / direction split is exact, and closed-form cases give their
known values (magnitude share, outlier residuals of appendix C, the token-scale
joint histogram of appendix B)."""
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


def test_residual_after_fixing_the_largest_errors():
    """Appendix C's curve: with all of the squared error in 1 % of the entries,
    fixing the top 1 % (or more) leaves nothing and fixing the rest leaves all;
    with equal errors everywhere the residual falls linearly in k."""
    x = torch.zeros(100, 128, dtype=torch.float64)
    xd = x.clone()
    xd[0, :] = 1.0                                      # 128 of 12800 entries
    r = bench.error_analysis(x + 1.0, xd + 1.0)["residual_sq_error_share"]
    for k in ("1pct", "5pct", "10pct", "25pct", "50pct"):
        assert r[k]["top_fixed"] == 0.0 and r[k]["bottom_fixed"] == 1.0
    assert abs(r["0.1pct"]["top_fixed"] - (1 - 13 / 128)) < 1e-12   # round(12.8) = 13 entries fixed
    u = bench.error_analysis(torch.ones(1000, 128, dtype=torch.float64), torch.full((1000, 128), 1.5,
                                                                                   dtype=torch.float64))
    for k in bench.TOPK_PCTS:
        assert abs(u["residual_sq_error_share"][f"{k:g}pct"]["top_fixed"] - (1 - k / 100)) < 1e-9
        assert abs(u["residual_sq_error_share"][f"{k:g}pct"]["bottom_fixed"] - k / 100) < 1e-9


def test_token_scale_joint_histogram():
    """Appendix B's joint distribution: exact reconstruction puts every token on
    the diagonal; doubling every token moves it two bins (one octave) up; a
    factor 1.5 (0.585 octaves) is off the diagonal by more than 0.5 and less
    than 1."""
    g = torch.Generator().manual_seed(9)
    x = torch.randn(3000, 128, generator=g, dtype=torch.float64) * torch.exp2(
        torch.rand(3000, 1, generator=g, dtype=torch.float64) * 3)          # log2 norms in [3.5, 6.5]
    h = bench.error_analysis(x, x)["token_scale_joint_hist"]
    c = torch.tensor(h["counts"])
    assert int(c.sum()) == 3000 and int(c.diagonal().sum()) == 3000
    h2 = bench.error_analysis(x, 2 * x)["token_scale_joint_hist"]
    c2 = torch.tensor(h2["counts"])
    assert int(c2.sum()) == 3000 and int(c2.diagonal(offset=2).sum()) == 3000
    off = bench.error_analysis(x, 1.5 * x)["token_scale_off_diagonal"]
    assert off["gt_0.1"] == off["gt_0.25"] == off["gt_0.5"] == 1.0 and off["gt_1"] == 0.0
