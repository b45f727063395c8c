"""A binary32 model of the HIP quantiser's arithmetic (test infrastructure).

The comparison protocol (parity.py) excuses metadata and code differences that
binary32 rounding can explain: ABS32 x max|Zn| for the rotation's absolute
error and TIE_REL32 x (|t| + 2|z|/s1) for the cancellation in t.  This module
re-runs the quantiser's steps in IEEE binary32 with numpy, in the kernel's
operation order where that order decides the rounding, so that a CPU test can
measure how far binary32 actually strays from the oracle's binary64 values and
check that the allowances cover it with margin:

* rotation, 16-bit inputs: each of the 16 channel groups is a sum of 16 exact
  +-x products accumulated in binary32 (the matrix-core half), then three
  butterfly stages over the 8 channels of a group in binary32;
  32-bit inputs: three in-lane butterfly stages, then four stages over the 16
  groups, every stage one binary32 add;
* normalisation: per lane, sequential FMAs over its 8 rows (channel step) or 8
  channels (token step), then the lane and wave trees of the kernel; one-pass
  moments, with the centred second pass where mean^2 > 16 var; the degenerate
  rule; reciprocal square roots with a seeded error of up to one ulp (the
  hardware's approximate instruction);
* metadata: power-of-two gauge, FP8 / FP16 encodings, Zn = y * rcp(s2) / sqrt(128);
* codes: t = fma(Zn, rcp(s1) / L, -z rcp(s1) / L), decided on L t.

It models the kernel; it is not the oracle and shares nothing with it.
"""
from __future__ import annotations

import numpy as np

N = 128
F32 = np.float32
F64 = np.float64
K_INV_SQRT_N = F32(1.0 / np.sqrt(128.0))
K_DEG_REL2 = F32(2.0 ** -32)
K_DEG_ABS2 = F32(2.0 ** -120)
K_CANCEL = F32(16.0)


def fma32(a, b, c):
    """binary32 fused multiply-add: the product is exact in binary64, one final rounding
    (the binary64 sum adds a second rounding only at exact binary32 midpoints)."""
    return (np.asarray(a, F32).astype(F64) * np.asarray(b, F32).astype(F64) + np.asarray(c, F32).astype(F64)).astype(F32)


class Approx:
    """Hardware reciprocal / reciprocal square root: the binary32 result within
    one ulp, perturbed by a seeded uniform error of up to one ulp."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)

    def _ulp(self, x64):
        x = x64.astype(F32)
        e = self.rng.integers(-1, 2, size=x.shape)
        return np.where(e > 0, np.nextafter(x, F32(np.inf)), np.where(e < 0, np.nextafter(x, F32(0)), x)).astype(F32)

    def rsq(self, v):
        v = np.asarray(v, F32).astype(F64)
        return self._ulp(1.0 / np.sqrt(np.where(v > 0, v, 1.0)))

    def rcp(self, v):
        return self._ulp(1.0 / np.asarray(v, F32).astype(F64))


def _fwht_last(v, n_bits, axis=-1):
    """In-place natural-order butterflies over the last axis's low n_bits index bits, in binary32."""
    v = np.moveaxis(v, axis, -1).copy()
    for s in range(n_bits):
        h = 1 << s
        idx = np.arange(v.shape[-1])
        lo = idx[(idx & h) == 0]
        a, b = v[..., lo].copy(), v[..., lo + h].copy()
        v[..., lo] = (a + b).astype(F32)
        v[..., lo + h] = (a - b).astype(F32)
    return np.moveaxis(v, -1, axis)


def rotate32(x, sixteen_bit):
    """sqrt(128) * (x H) in binary32 for x [n][128][128] (float64 holding the input values)."""
    x = np.asarray(x, F64)
    n = x.shape[0]
    if sixteen_bit:
        xg = x.reshape(n, N, 16, 8)                       # [tile][token][group g'][j]
        y = np.zeros((n, N, 16, 8), F32)                   # [tile][token][output group][j]
        order = [4 * i + q for q in range(4) for i in range(4)]   # matrix-core K slot order
        for go in range(16):
            acc = np.zeros((n, N, 8), F32)
            for gi in order:
                sgn = -1.0 if bin(gi & go).count("1") & 1 else 1.0
                acc = (acc.astype(F64) + sgn * xg[:, :, gi, :]).astype(F32)
            y[:, :, go, :] = acc
        y = _fwht_last(y, 3)                               # H8 over j
        return y.reshape(n, N, N)
    y = x.astype(F32).reshape(n, N, 16, 8)
    y = _fwht_last(y, 3)                                   # 8 channels in-lane
    y = _fwht_last(y, 4, axis=2)                           # 16 groups
    return y.reshape(n, N, N)


def _col_sums(w_rows, m):
    """Channel-step sums of w_i * m_ij over the 128 rows, in the kernel's order:
    sequential FMAs over a lane's 8 rows, then lane bit 5, lane bit 4, then the
    four waves pairwise.  w_rows [n][128], m [n][128][128] -> [n][128]."""
    n = m.shape[0]
    mb = m.reshape(n, 4, 4, 8, N)                          # wave, row group, a, column
    wb = w_rows.reshape(n, 4, 4, 8, 1)
    s = np.zeros((n, 4, 4, N), F32)
    for a in range(8):
        s = fma32(wb[:, :, :, a], mb[:, :, :, a], s)
    s = np.stack([(s[:, :, 0] + s[:, :, 2]).astype(F32), (s[:, :, 1] + s[:, :, 3]).astype(F32)], 2)
    s = (s[:, :, 0] + s[:, :, 1]).astype(F32)              # [n][wave][col]
    return ((s[:, 0] + s[:, 1]).astype(F32) + (s[:, 2] + s[:, 3]).astype(F32)).astype(F32)


def _row_sums(w_cols, m):
    """Token-step sums of w_j * m_ij over the 128 channels: sequential FMAs over a
    lane's 8 channels, then a pairwise tree over the 16 lanes of the row."""
    n = m.shape[0]
    mb = m.reshape(n, N, 16, 8)
    wb = w_cols.reshape(n, 1, 16, 8)
    s = np.zeros((n, N, 16), F32)
    for j in range(8):
        s = fma32(wb[..., j], mb[..., j], s)
    idx = np.arange(16)
    for x in (8, 7, 2, 1):
        s = (s + s[..., idx ^ x]).astype(F32)
    return s[..., 0]


def _sum32(v, axis=-1):
    return np.sum(np.asarray(v, F32), axis=axis, dtype=F32)


def fp8_code(v):
    """OCP E4M3 code of non-negative binary32 v, round to nearest even, saturating at 448."""
    v = np.asarray(v, F32)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0).astype(F64))).astype(np.int64)
    sub = e < -6
    code_sub = np.rint(v.astype(F64) * 512.0)
    m = np.rint(v.astype(F64) * np.exp2(3.0 - e))
    code_n = (e + 7) * 8 + m - 8
    code = np.where(sub, code_sub, np.minimum(code_n, 0x7E))
    return np.where(v > 0, code, 0).astype(np.int64)


def fp8_value(code):
    code = np.asarray(code, np.int64)
    e, m = (code >> 3) & 15, code & 7
    return np.where(e == 0, m / 512.0, (8 + m) * np.exp2(e - 10.0)).astype(F32)


def quantize32(x, sixteen_bit, bits, axis, n_iter=8, seed=0):
    """Model of one quantise launch.  Returns a dict of binary32 quantities:
    g (gauge-fixed second-scale factor before FP8), s2 codes, s1_pre, z_pre
    (before FP8 / FP16), s1 codes, z (FP16 bits), the t on which each code is
    decided (L * fl(fma(...)), unclamped), and the rotated y / sqrt(128)."""
    ap = Approx(seed)
    L = (1 << bits) - 1
    y = rotate32(x, sixteen_bit)
    n = y.shape[0]
    y2 = (y * y).astype(F32)
    wr = np.ones((n, N), F32)
    wr2 = np.ones((n, N), F32)
    colsq = None
    last_rvar = last_rms2r = None
    gc = None

    def channel_moments(first):
        nonlocal colsq
        s = _col_sums(wr, y)
        q = _col_sums(wr2, y2)
        if first:
            colsq = q
        rms2 = (_sum32(q) * F32(1.0 / 16384.0)).astype(F32)
        mean = (s * F32(1.0 / 128.0)).astype(F32)
        var = fma32(-mean, mean, (q * F32(1.0 / 128.0)).astype(F32))
        redo = np.any(mean * mean > K_CANCEL * var, axis=1)
        if redo.any():
            d = fma32(wr[:, :, None], y, -mean[:, None, :])
            q2 = _col_sums(np.ones((n, N), F32), (d * d).astype(F32))
            var = np.where(redo[:, None], (q2 * F32(1.0 / 128.0)).astype(F32), var)
        return var, rms2

    n_full = n_iter - 1 if (axis == 1 and n_iter > 0) else n_iter
    for it in range(n_full):
        var, rms2 = channel_moments(it == 0)
        thr = (K_DEG_REL2 * rms2).astype(F32)[:, None]
        floor2 = F32(K_DEG_ABS2 * 128)
        fb = np.where(rms2 >= floor2, ap.rsq(rms2), K_INV_SQRT_N)[:, None]
        f = np.where((var > thr) & (var >= floor2), ap.rsq(var), fb).astype(F32)
        wc, wc2 = f, (f * f).astype(F32)
        rms2r = (_sum32(fma32(colsq, wc2, 0.0)) * F32(1.0 / 16384.0)).astype(F32)
        s = _row_sums(wc, y)
        q = _row_sums(wc2, y2)
        rmean = (s * F32(1.0 / 128.0)).astype(F32)
        rvar = fma32(-rmean, rmean, (q * F32(1.0 / 128.0)).astype(F32))
        redo = np.any((rmean * rmean > K_CANCEL * rvar).reshape(n, 4, 32), axis=2)   # per wave of 32 rows
        if redo.any():
            d = fma32(wc[:, None, :], y, -rmean[:, :, None])
            q2 = _row_sums(np.ones((n, N), F32), (d * d).astype(F32))
            rvar = np.where(np.repeat(redo, 32, axis=1), (q2 * F32(1.0 / 128.0)).astype(F32), rvar)
        fbr = np.where(rms2r >= K_DEG_ABS2, ap.rsq(rms2r), F32(1.0))[:, None]
        fr = np.where((rvar > (K_DEG_REL2 * rms2r)[:, None]) & (rvar >= K_DEG_ABS2), ap.rsq(rvar), fbr).astype(F32)
        last_rvar, last_rms2r = rvar, rms2r
        wr, wr2 = fr, (fr * fr).astype(F32)
    if axis == 1 and n_iter > 0:
        var, rms2 = channel_moments(n_iter == 1)
        thr = (K_DEG_REL2 * rms2)[:, None]
        floor2 = F32(K_DEG_ABS2 * 128)
        ok = (var > thr) & (var >= floor2)
        gc = np.where(ok, np.sqrt((var * F32(1.0 / 128.0)).astype(F32)),
                      np.where(rms2 >= floor2, np.sqrt((rms2 * F32(1.0 / 128.0)).astype(F32)), 1.0)[:, None])
        gvec = gc.astype(F32)
    elif axis == 1:
        gvec = np.ones((n, N), F32)
    elif n_iter > 0:
        ok = (last_rvar > (K_DEG_REL2 * last_rms2r)[:, None]) & (last_rvar >= K_DEG_ABS2)
        gvec = np.where(ok, np.sqrt(last_rvar), np.where(last_rms2r >= K_DEG_ABS2, np.sqrt(last_rms2r), 1.0)[:, None])
        gvec = gvec.astype(F32)
    else:
        gvec = np.ones((n, N), F32)

    # gauge: frexp exponent of the binary32 mean
    gmean = (_sum32(gvec) * F32(1.0 / 128.0)).astype(F32)
    gexp = np.clip(((gmean.view(np.uint32) >> 23) & 255).astype(np.int64) - 126, -126, 126)
    g = (gvec * np.exp2(-gexp.astype(F64))[:, None].astype(F32)).astype(F32)
    s2c = np.maximum(fp8_code(g), 1)
    m = (ap.rcp(fp8_value(s2c)) * K_INV_SQRT_N).astype(F32)
    zn = (y * (m[:, :, None] if axis == 0 else m[:, None, :])).astype(F32)
    gaxis = 1 if axis == 0 else 2                          # reduce over tokens (K groups = channels) or channels
    mn, mx = zn.min(gaxis), zn.max(gaxis)
    s1_pre = ((mx - mn).astype(F32) * F32(1.0 / L)).astype(F32)
    s1c = np.maximum(fp8_code(s1_pre), 1)
    zsat = np.clip(mn, -65504.0, 65504.0).astype(F32)
    zb = zsat.astype(np.float16)
    is1 = (ap.rcp(fp8_value(s1c)) * F32(1.0 / L)).astype(F32)
    zoff = (-zb.astype(F32) * is1).astype(F32)
    sh = (lambda a: a[:, None, :]) if axis == 0 else (lambda a: a[:, :, None])
    t = L * fma32(zn, sh(is1), sh(zoff)).astype(F64)
    return dict(g=g, s2=s2c.astype(np.uint8), s1_pre=s1_pre, s1=s1c.astype(np.uint8), z_pre=mn, z=zb.view(np.uint16),
                t=t, y=y.astype(F64) / np.sqrt(128.0))


def records(res, bits):
    """Packed-record stand-ins carrying the model's metadata (codes left zero)."""
    n = res["s2"].shape[0]
    c = 2048 * bits
    rec = np.zeros((n, c + 512), np.uint8)
    rec[:, c:c + 128] = res["s1"]
    rec[:, c + 128:c + 256] = res["s2"]
    rec[:, c + 256:c + 512] = np.ascontiguousarray(res["z"]).view(np.uint8).reshape(n, 256)
    return rec
