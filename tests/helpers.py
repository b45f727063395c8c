"""Small helpers shared by the tests (no codec arithmetic here)."""
import numpy as np
import scipy.linalg

N = 128


def hadamard_ref():
    """Orthonormal Sylvester Hadamard matrix from scipy (a library routine)."""
    return scipy.linalg.hadamard(N).astype(np.float64) / np.sqrt(N)


def f16_bits(a):
    return np.ascontiguousarray(np.asarray(a, np.float16)).view(np.uint16)


def fp8_values():
    """(codes, values) of all finite non-negative FP8 E4M3 numbers, via torch's decoder."""
    import torch

    codes = torch.arange(128, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).double().numpy()
    keep = np.isfinite(vals)
    return codes.numpy()[keep], vals[keep]


def nearest_fp8(x):
    """Nearest FP8 E4M3 value to each x >= 0, ties to the even code, saturating at 448 (brute force)."""
    codes, vals = fp8_values()
    x = np.atleast_1d(np.asarray(x, np.float64))
    d = np.abs(vals[None, :] - x[:, None])
    out = np.empty_like(x)
    for i in range(len(x)):
        best = np.flatnonzero(d[i] == d[i].min())
        pick = best[0]
        if len(best) == 2 and codes[best[0]] % 2 == 1:
            pick = best[1]
        out[i] = vals[pick]
    return out


def code_position(bits, axis, t, c):
    """Byte and bit of the code of token t, channel c in the documented record
    layout (include/kvarn.h): row r = s2 index, position p = group index."""
    r, p = (t, c) if axis == 0 else (c, t)
    n, i = r // 8, r % 8
    if bits == 2:
        return 1024 * (i // 2) + 16 * (16 * (p // 32) + n) + 8 * (i % 2) + (p % 32) // 4, 2 * (p % 4)
    return 1024 * i + 16 * (16 * ((p // 16) % 4) + n) + 8 * (p // 64) + (p % 16) // 2, 4 * (p % 2)


def set_code(record, bits, axis, t, c, code):
    """Overwrite the code of token t, channel c of one packed record in place."""
    byte, bit = code_position(bits, axis, t, c)
    mask = (2 ** bits - 1) << bit
    record[byte] = (int(record[byte]) & (0xFF ^ mask)) | ((int(code) << bit) & mask)


def tiles_bits(tiles_f16):
    """float16 array [..., 128, 128] -> uint16 bits, flattened to [n][128][128]."""
    a = np.ascontiguousarray(np.asarray(tiles_f16, np.float16))
    return a.view(np.uint16).reshape(-1, N, N)


def rel_spread(v):
    v = np.asarray(v, np.float64)
    return (v.max() - v.min()) / np.mean(np.abs(v))
