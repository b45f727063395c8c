"""Comparison protocol between the HIP codec and the oracle (test infrastructure).

The oracle computes in binary64, the kernels in binary32, so a value that lands
within rounding noise of a rounding midpoint may round the other way.  The
protocol therefore compares in dependency order and only excuses a difference
where the oracle's own unrounded value sits at such a midpoint:

1. s2: the GPU's FP8 second scale equals the oracle's, or is the other of the
   two FP8 neighbours of the oracle's unrounded value and that value is within
   REL_META of their midpoint.
2. s1, z: recomputed by the oracle *with the GPU's s2*; same rule (FP8 / FP16).
3. codes: recomputed by the oracle *with the GPU's s1, s2, z*; a code may differ
   by exactly one level only where the oracle's t = (Zn - z) / s1 is within
   TIE_ABS (+ a term for binary32 cancellation) of k + 1/2.
4. the raw fraction of identical codes between the two records is reported and
   must be at least 99.99 %.

Any difference outside these classes is "unexplained" and fails the test.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

N = 128
REL_META = 1e-4
TIE_ABS = 1e-4
TIE_REL32 = 4e-6


def fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _fp8_neighbours(x):
    """The two FP8 values bracketing x (x >= 0) from the full table."""
    table = fp8_values(np.arange(127, dtype=np.uint8))  # finite non-negative codes 0..126
    hi = np.searchsorted(table, x, side="left").clip(1, len(table) - 1)
    return table[hi - 1], table[hi]


def _f16_neighbours(x):
    lo = x.astype(np.float16)
    lo64 = lo.astype(np.float64)
    other = np.where(lo64 > x, np.nextafter(lo, np.float16(-np.inf)), np.nextafter(lo, np.float16(np.inf)))
    return np.minimum(lo64, other.astype(np.float64)), np.maximum(lo64, other.astype(np.float64))


def meta_ok(gpu_vals, pre, kind, floor=None, scale=None):
    """Mask of GPU metadata values that are the oracle's rounding of `pre`, or the
    other neighbour when `pre` sits within tolerance of the midpoint."""
    pre = np.asarray(pre, np.float64)
    if kind == "fp8":
        ref = np.array([oracle.fp8_round(v) for v in pre.reshape(-1)]).reshape(pre.shape)
        lo, hi = _fp8_neighbours(np.abs(pre))
    else:
        ref = np.array([oracle.f16_round(v) for v in pre.reshape(-1)]).reshape(pre.shape)
        lo, hi = _f16_neighbours(pre)
    if floor is not None:
        ref = np.maximum(ref, floor)
    mid = (lo + hi) / 2
    tol = REL_META * (np.abs(pre) if scale is None else scale)
    near = np.abs(pre - mid) <= tol
    flipped = ((gpu_vals == lo) | (gpu_vals == hi)) & near
    if floor is not None:
        flipped |= (gpu_vals == floor) & (pre <= floor * (1 + REL_META))
    return (gpu_vals == ref) | flipped


class Report(dict):
    def __str__(self):
        return ", ".join(f"{k}={v}" for k, v in self.items())


def compare_quantize(view: "oracle.TileView", bits: int, axis: int, gpu_rec: np.ndarray, n_iter: int = 8) -> Report:
    """Run the full protocol for the tiles of `view` against GPU records [n][Pb]."""
    gpu_rec = np.ascontiguousarray(gpu_rec, np.uint8)
    L = 2 ** bits - 1
    ref_rec, dbg = oracle.quantize(view, bits, axis, n_iter=n_iter, debug=True)
    gc, g1, g2, gz = oracle.record_fields(gpu_rec, bits)
    rc, r1, r2, rz = oracle.record_fields(ref_rec, bits)
    rep = Report(tiles=view.n)

    # 1. second scale (with the power-of-two gauge: a whole-tile binade shift is a gauge flip)
    s2_gpu = fp8_values(g2)
    ok2 = meta_ok(s2_gpu, dbg["g_pre"], "fp8", floor=2.0 ** -9)
    gmean = dbg["g_pre"].mean(1)
    gauge_edge = (np.abs(gmean - 0.5) <= REL_META) | (np.abs(gmean - 1.0) <= REL_META)
    for n in np.flatnonzero(~ok2.all(1) & gauge_edge):
        for f in (2.0, 0.5):
            alt = meta_ok(s2_gpu[n], dbg["g_pre"][n] * f, "fp8", floor=2.0 ** -9)
            if alt.all():
                ok2[n] = True
    rep["s2_equal"] = int((g2 == r2).sum())
    rep["s2_flips"] = int((ok2 & (g2 != r2)).sum())
    rep["s2_bad"] = int((~ok2).sum())

    # 2. group scale and zero-point, given the GPU's s2
    s1_pre, z_pre = oracle.group_meta_given_s2(view, bits, axis, g2)
    s1_gpu = fp8_values(g1)
    z_gpu = gz.view(np.float16).astype(np.float64)
    scale = (2 * np.abs(z_pre) + L * s1_pre) / L
    ok1 = meta_ok(s1_gpu, s1_pre, "fp8", floor=2.0 ** -9, scale=scale)
    okz = meta_ok(z_gpu, np.clip(z_pre, -65504, 65504), "f16", scale=np.abs(z_pre) + L * s1_pre)
    rep["s1_flips"] = int((ok1 & (g1 != r1)).sum())
    rep["z_flips"] = int((okz & (gz != rz)).sum())
    rep["s1_bad"] = int((~ok1).sum())
    rep["z_bad"] = int((~okz).sum())

    # 3. codes, given all of the GPU's metadata
    codes_ref, t = oracle.codes_given_meta(view, bits, axis, gpu_rec)
    codes_gpu = oracle.unpack_codes(gpu_rec, bits)
    diff = codes_gpu.astype(np.int64) - codes_ref.astype(np.int64)
    s1g = s1_gpu[:, None, :] if axis == 0 else s1_gpu[:, :, None]
    zg = z_gpu[:, None, :] if axis == 0 else z_gpu[:, :, None]
    tol = TIE_ABS + TIE_REL32 * (np.abs(t) + 2 * np.abs(zg) / s1g)
    tie = np.abs(np.abs(t - np.floor(t)) - 0.5) <= tol
    rep["code_ties"] = int(((diff != 0) & (np.abs(diff) == 1) & tie).sum())
    rep["code_bad"] = int(((diff != 0) & ~((np.abs(diff) == 1) & tie)).sum())

    # 4. raw agreement of the packed records
    raw_codes = oracle.unpack_codes(ref_rec, bits)
    rep["raw_identical_codes"] = float((raw_codes == codes_gpu).mean())
    rep["records_identical"] = int((gpu_rec == ref_rec).all(1).sum())
    rep["unexplained"] = rep["s2_bad"] + rep["s1_bad"] + rep["z_bad"] + rep["code_bad"]
    return rep


def assert_quantize_parity(rep: Report, min_identical: float = 0.9999):
    assert rep["unexplained"] == 0, str(rep)
    assert rep["raw_identical_codes"] >= min_identical, str(rep)


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Exact bit patterns of a 16-bit torch tensor as uint16 numpy (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dequant_fp32_error(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-element error relative to each tile's RMS."""
    rms = np.sqrt((ref.reshape(ref.shape[0], -1) ** 2).mean(1))
    rms = np.where(rms > 0, rms, 1.0)
    err = np.abs(gpu.astype(np.float64) - ref).reshape(ref.shape[0], -1).max(1)
    return float((err / rms).max())


def rounded_output_ok(gpu: torch.Tensor, ref: np.ndarray, abs_tol=0.0) -> np.ndarray:
    """A 16-bit GPU output equals the round-to-nearest-even of the oracle value, or is
    its other neighbour where the oracle value is within 1e-5 (relative) + abs_tol of
    the midpoint.  abs_tol covers the binary32 error of the inverse rotation, which is
    absolute (a few 1e-7 of the tile RMS), so it matters for near-zero outputs."""
    dt = gpu.dtype
    ref64 = np.clip(ref, -65504, 65504) if dt == torch.float16 else ref
    ref_t = torch.from_numpy(np.ascontiguousarray(ref64, np.float64))
    exp = ref_t.to(dt)
    g = gpu.cpu()
    eb = exp.view(torch.int16).to(torch.int32) & 0xFFFF
    sign, mag = eb & 0x8000, eb & 0x7FFF
    away = sign | (mag + 1)                                   # one ulp further from zero
    toward = torch.where(mag > 0, sign | (mag - 1), (sign ^ 0x8000) | 1)
    e64 = exp.double()
    other_bits = torch.where(ref_t.abs() > e64.abs(), away, toward)
    other_bits = torch.where(other_bits >= 0x8000, other_bits - 0x10000, other_bits).to(torch.int16)
    other = other_bits.view(dt)
    mid = (e64 + other.double()) / 2
    near = (ref_t - mid).abs() <= 1e-5 * ref_t.abs() + torch.as_tensor(abs_tol, dtype=torch.float64)
    return ((g == exp) | ((g == other) & near)).numpy()


def tile_rms(ref: np.ndarray) -> np.ndarray:
    """RMS of each tile of ref [n][128][128], broadcastable against it."""
    return np.sqrt((ref.reshape(ref.shape[0], -1) ** 2).mean(1))[:, None, None]


def rel_l2_rows(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    g = gpu.reshape(-1, N).astype(np.float64)
    r = ref.reshape(-1, N)
    den = np.linalg.norm(r, axis=1)
    return np.linalg.norm(g - r, axis=1) / np.where(den > 0, den, 1.0)
