"""Comparison protocol between the HIP codec and the oracle (test infrastructure).

The oracle computes in binary64, the kernels in binary32, so a value that lands
within rounding noise of a rounding boundary may round the other way.  The
protocol compares in dependency order and only excuses a difference that the
oracle's own unrounded value explains:

1. s2: the GPU's FP8 second scale is the rounding of some value within
   delta = REL_META * g of the oracle's unrounded gauge-fixed factor g (a whole
   tile shifted by one binade is accepted when the gauge mean sits within
   REL_META of a power of two).
2. s1, z: recomputed by the oracle *with the GPU's s2*; the GPU's value must be
   the rounding of some value within delta of the oracle's unrounded one, with
   delta = REL_META * |value| + ABS32 * max|Zn| of the tile.  The absolute part is
   the binary32 error of the rotation, which is absolute: channels that are zero
   in exact arithmetic carry ~1e-7 of the tile's magnitude on the GPU.
3. codes: recomputed by the oracle *with the GPU's s1, s2, z*; a code may differ
   by exactly one level only where the oracle's t = (Zn - z) / s1 is within
   TIE_ABS + TIE_REL32 (|t| + 2|z|/s1) + ABS32 max|Zn| / s1 of k + 1/2.
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
# Binary32 parts of the windows.  A binary32 model of the quantiser's own
# operation order (emu32.py) strays from the oracle by at most ~0.22 of these on
# the edge tiles and the workload samples (test_binary32_allowances.py), so the
# window is about four times what the kernel's arithmetic can produce.
TIE_REL32 = 1e-6
ABS32 = 1.2e-6
FP8_FLOOR = 2.0 ** -9


def fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _round(kind, v):
    v = np.asarray(v, np.float64)
    f = oracle.fp8_round if kind == "fp8" else oracle.f16_round
    return np.array([f(x) for x in v.reshape(-1)]).reshape(v.shape)


def meta_ok(gpu_vals, pre, kind, delta, floor=None):
    """GPU metadata value lies between the roundings of pre - delta and pre + delta."""
    pre = np.asarray(pre, np.float64)
    lo = _round(kind, pre - delta)
    hi = _round(kind, pre + delta)
    if floor is not None:
        lo, hi = np.maximum(lo, floor), np.maximum(hi, floor)
    return (gpu_vals >= lo) & (gpu_vals <= hi)


class Report(dict):
    def __str__(self):
        return ", ".join(f"{k}={v}" for k, v in self.items())


def compare_quantize(view: "oracle.TileView", bits: int, axis: int, gpu_rec: np.ndarray, n_iter: int = 8,
                     rotate: bool = True) -> Report:
    """Run the full protocol for the tiles of `view` against GPU records [n][Pb]."""
    gpu_rec = np.ascontiguousarray(gpu_rec, np.uint8)
    L = 2 ** bits - 1
    ref_rec, dbg = oracle.quantize(view, bits, axis, n_iter=n_iter, rotate=rotate, debug=True)
    gc, g1, g2, gz = oracle.record_fields(gpu_rec, bits)
    rc, r1, r2, rz = oracle.record_fields(ref_rec, bits)
    rep = Report(tiles=view.n)

    # 1. second scale (with the power-of-two gauge: a whole-tile binade shift is a gauge flip)
    s2_gpu = fp8_values(g2)
    ok2 = meta_ok(s2_gpu, dbg["g_pre"], "fp8", REL_META * dbg["g_pre"], floor=FP8_FLOOR)
    gmean = dbg["g_pre"].mean(1)
    gauge_edge = (np.abs(gmean - 0.5) <= REL_META) | (np.abs(gmean - 1.0) <= REL_META)
    for n in np.flatnonzero(~ok2.all(1) & gauge_edge):
        for f in (2.0, 0.5):
            pre = dbg["g_pre"][n] * f
            if meta_ok(s2_gpu[n], pre, "fp8", REL_META * pre, floor=FP8_FLOOR).all():
                ok2[n] = True
    rep["s2_equal"] = int((g2 == r2).sum())
    rep["s2_flips"] = int((ok2 & (g2 != r2)).sum())
    rep["s2_bad"] = int((~ok2).sum())

    # magnitude of Zn = Y / s2 per tile (GPU's s2), for the absolute binary32 allowance
    y = dbg["y"]
    zn = y / (s2_gpu[:, :, None] if axis == 0 else s2_gpu[:, None, :])
    zmax = np.abs(zn).reshape(view.n, -1).max(1)[:, None]

    # 2. group scale and zero-point, given the GPU's s2
    s1_pre, z_pre = oracle.group_meta_given_s2(view, bits, axis, g2, rotate=rotate)
    s1_gpu = fp8_values(g1)
    z_gpu = gz.view(np.float16).astype(np.float64)
    ok1 = meta_ok(s1_gpu, s1_pre, "fp8", REL_META * s1_pre + 2 * ABS32 * zmax / L, floor=FP8_FLOOR)
    okz = meta_ok(z_gpu, np.clip(z_pre, -65504, 65504), "f16", REL_META * np.abs(z_pre) + ABS32 * zmax)
    rep["s1_flips"] = int((ok1 & (g1 != r1)).sum())
    rep["z_flips"] = int((okz & (gz != rz)).sum())
    rep["s1_bad"] = int((~ok1).sum())
    rep["z_bad"] = int((~okz).sum())

    # 3. codes, given all of the GPU's metadata
    codes_ref, t = oracle.codes_given_meta(view, bits, axis, gpu_rec, rotate=rotate)
    codes_gpu = oracle.unpack_codes(gpu_rec, bits, axis)
    diff = codes_gpu.astype(np.int64) - codes_ref.astype(np.int64)
    s1g = s1_gpu[:, None, :] if axis == 0 else s1_gpu[:, :, None]
    zg = z_gpu[:, None, :] if axis == 0 else z_gpu[:, :, None]
    tol = TIE_ABS + TIE_REL32 * (np.abs(t) + 2 * np.abs(zg) / s1g) + ABS32 * zmax[:, :, None] / s1g
    tie = np.abs(np.abs(t - np.floor(t)) - 0.5) <= tol
    rep["code_ties"] = int(((diff != 0) & (np.abs(diff) == 1) & tie).sum())
    rep["code_bad"] = int(((diff != 0) & ~((np.abs(diff) == 1) & tie)).sum())

    # 4. raw agreement of the packed records
    raw_codes = oracle.unpack_codes(ref_rec, bits, axis)
    rep["raw_identical_codes"] = float((raw_codes == codes_gpu).mean())
    rep["records_identical"] = int((gpu_rec == ref_rec).all(1).sum())
    rep["unexplained"] = rep["s2_bad"] + rep["s1_bad"] + rep["z_bad"] + rep["code_bad"]
    return rep


_SUMMED = ("s2_equal", "s2_flips", "s2_bad", "s1_flips", "z_flips", "s1_bad", "z_bad", "code_ties", "code_bad",
           "records_identical", "unexplained")


def compare_quantize_many(tiles: np.ndarray, dtype: int, bits: int, axis: int, gpu_rec: np.ndarray,
                          n_iter: int = 8, rotate: bool = True, chunk: int = 512) -> Report:
    """compare_quantize for many dense tiles [n][128][128] (16-bit bits or
    float32).  A record byte-identical to the oracle's passes every step of the
    protocol trivially, so only the records that differ go through it (in chunks
    of at most `chunk` tiles); the counts are those of the full protocol."""
    gpu_rec = np.ascontiguousarray(gpu_rec, np.uint8)
    tiles = np.ascontiguousarray(tiles).reshape(-1, N, N)
    n = tiles.shape[0]
    ref = oracle.quantize(oracle.TileView.dense(tiles, dtype), bits, axis, n_iter=n_iter, rotate=rotate)
    same = (gpu_rec == ref).all(1)
    rep = Report(tiles=n, full_protocol_tiles=int((~same).sum()))
    for k in _SUMMED:
        rep[k] = 0
    rep["s2_equal"] = N * int(same.sum())
    rep["records_identical"] = int(same.sum())
    identical_codes = float(same.sum()) * N * N
    diff = np.flatnonzero(~same)
    for c0 in range(0, diff.size, chunk):
        idx = diff[c0:c0 + chunk]
        sub = compare_quantize(oracle.TileView.dense(tiles[idx], dtype), bits, axis, gpu_rec[idx], n_iter=n_iter,
                               rotate=rotate)
        for k in _SUMMED:
            rep[k] += sub[k]
        identical_codes += sub["raw_identical_codes"] * idx.size * N * N
    rep["raw_identical_codes"] = identical_codes / (n * N * N) if n else 1.0
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
    """A 16-bit GPU output is the round-to-nearest-even of some value within
    delta = 1e-5 |ref| + abs_tol of the oracle value ref, i.e. it lies between
    RNE(ref - delta) and RNE(ref + delta).  With delta -> 0 this is exact RNE; the
    relative part allows the other neighbour at a midpoint, abs_tol covers the
    binary32 error of the inverse rotation, which is absolute (a few 1e-7 of the
    tile RMS) and dominates for outputs that are zero in exact arithmetic."""
    dt = gpu.dtype
    clip = (lambda a: np.clip(a, -65504, 65504)) if dt == torch.float16 else (lambda a: a)
    delta = 1e-5 * np.abs(ref) + abs_tol
    lo = torch.from_numpy(np.ascontiguousarray(clip(ref - delta), np.float64)).to(dt).double()
    hi = torch.from_numpy(np.ascontiguousarray(clip(ref + delta), np.float64)).to(dt).double()
    g = gpu.cpu().double()
    return ((g >= lo) & (g <= hi)).numpy()


def tile_rms(ref: np.ndarray) -> np.ndarray:
    """RMS of each tile of ref [n][128][128], broadcastable against it."""
    return np.sqrt((ref.reshape(ref.shape[0], -1) ** 2).mean(1))[:, None, None]


def rel_l2_rows(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    g = gpu.reshape(-1, N).astype(np.float64)
    r = ref.reshape(-1, N)
    den = np.linalg.norm(r, axis=1)
    return np.linalg.norm(g - r, axis=1) / np.where(den > 0, den, 1.0)
