"""CPU oracle for the KVarN KV-cache tile codec -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never does, and the two share no code.

The arithmetic lives in ``kvarn_oracle.c`` (plain C, binary64, OpenMP over
tiles); this module only marshals numpy arrays through ctypes.  See the header
of ``kvarn_oracle.c`` for the algorithm, the record layout and the sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvarn_oracle.c")
_LIB = os.path.join(_HERE, "libkvarn_oracle.so")

DT_F16, DT_BF16, DT_F32 = 0, 1, 2
AXIS_K, AXIS_V = 0, 1
N = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libkvarn_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.kvo_bf16_decode.restype = D
        L.kvo_bf16_decode.argtypes = [ctypes.c_uint16]
        L.kvo_f16_decode.restype = D
        L.kvo_f16_decode.argtypes = [ctypes.c_uint16]
        L.kvo_fp8_decode.restype = D
        L.kvo_fp8_decode.argtypes = [ctypes.c_uint8]
        L.kvo_fp8_round.restype = D
        L.kvo_fp8_round.argtypes = [D]
        L.kvo_fp8_encode.restype = ctypes.c_uint8
        L.kvo_fp8_encode.argtypes = [D]
        L.kvo_f16_round.restype = D
        L.kvo_f16_round.argtypes = [D]
        L.kvo_f16_encode.restype = ctypes.c_uint16
        L.kvo_f16_encode.argtypes = [D]
        L.kvo_record_bytes.restype = ctypes.c_size_t
        L.kvo_record_bytes.argtypes = [I]
        L.kvo_hadamard.restype = None
        L.kvo_hadamard.argtypes = [P]
        L.kvo_sinkhorn.restype = None
        L.kvo_sinkhorn.argtypes = [P, I, P, P]
        L.kvo_quantize_tiles.restype = I
        L.kvo_quantize_tiles.argtypes = [P, I, I64, I64, I64, P, I, I, I, I, P, P, P, P, P]
        L.kvo_group_meta_given_s2.restype = I
        L.kvo_group_meta_given_s2.argtypes = [P, I, I64, I64, I64, P, I, I, I, P, P, P]
        L.kvo_codes_given_meta.restype = I
        L.kvo_codes_given_meta.argtypes = [P, I, I64, I64, I64, P, I, I, I, P, P, P]
        L.kvo_unpack_codes.restype = I
        L.kvo_unpack_codes.argtypes = [P, I64, I, I, P]
        L.kvo_dequantize_tiles.restype = I
        L.kvo_dequantize_tiles.argtypes = [P, I64, I, I, I, P]
        L.kvo_decode_attn.restype = I
        L.kvo_decode_attn.argtypes = [P, P, P, P, P, I64, I, I, I, I, I, I, D, P, P, I, P, P, P, I, P]
        L.kvo_num_threads.restype = I
        L.kvo_num_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def record_bytes(bits: int) -> int:
    return int(lib().kvo_record_bytes(bits))


def num_threads() -> int:
    return int(lib().kvo_num_threads())


# --------------------------------------------------------------------------- formats
fp8_decode = lambda b: lib().kvo_fp8_decode(int(b))  # noqa: E731
fp8_round = lambda v: lib().kvo_fp8_round(float(v))  # noqa: E731
fp8_encode = lambda v: int(lib().kvo_fp8_encode(float(v)))  # noqa: E731
f16_decode = lambda b: lib().kvo_f16_decode(int(b))  # noqa: E731
f16_round = lambda v: lib().kvo_f16_round(float(v))  # noqa: E731
f16_encode = lambda v: int(lib().kvo_f16_encode(float(v)))  # noqa: E731
bf16_decode = lambda b: lib().kvo_bf16_decode(int(b))  # noqa: E731


def hadamard() -> np.ndarray:
    h = np.empty((N, N), np.float64)
    lib().kvo_hadamard(_ptr(h))
    return h


def sinkhorn(y: np.ndarray, n_iter: int = 8):
    """Per-token r and per-channel c of one rotated tile y[128 tokens][128 ch]."""
    y = np.ascontiguousarray(y, np.float64)
    assert y.shape == (N, N)
    r = np.empty(N, np.float64)
    c = np.empty(N, np.float64)
    lib().kvo_sinkhorn(_ptr(y), n_iter, _ptr(r), _ptr(c))
    return r, c


# --------------------------------------------------------------------------- tiles
class TileView:
    """Element addressing of a batch of tiles inside a flat buffer.

    ``buf`` is a flat numpy array (uint16 holding fp16 or bf16 bits, or
    float32).  Tile i starts at ``offsets[i]`` (or ``i * tile_stride``); token t,
    channel c is element ``start + t * token_stride + c``.
    """

    def __init__(self, buf, dtype, n_tiles, tile_stride=N * N, token_stride=N, offsets=None):
        self.buf = np.ascontiguousarray(buf).reshape(-1)
        self.dtype = dtype
        self.n = int(n_tiles)
        self.tile_stride = int(tile_stride)
        self.token_stride = int(token_stride)
        self.offsets = None if offsets is None else np.ascontiguousarray(offsets, np.int64)

    @classmethod
    def dense(cls, tiles, dtype):
        """tiles: array [..., 128, 128] (uint16 bits or float32)."""
        a = np.ascontiguousarray(tiles)
        n = a.size // (N * N)
        return cls(a.reshape(-1), dtype, n)

    def args(self):
        return (_ptr(self.buf), self.dtype, self.n, self.tile_stride, self.token_stride, _ptr(self.offsets))


def quantize(view: TileView, bits: int, axis: int, n_iter: int = 8, rotate: bool = True, debug: bool = False):
    """Packed records [n][Pb] uint8 (plus pre-rounding values when debug)."""
    n = view.n
    rec = np.zeros((n, record_bytes(bits)), np.uint8)
    g_pre = s1_pre = z_pre = y = None
    if debug:
        g_pre = np.empty((n, N), np.float64)
        s1_pre = np.empty((n, N), np.float64)
        z_pre = np.empty((n, N), np.float64)
        y = np.empty((n, N, N), np.float64)
    rc = lib().kvo_quantize_tiles(*view.args(), bits, axis, n_iter, int(rotate), _ptr(rec), _ptr(g_pre),
                                  _ptr(s1_pre), _ptr(z_pre), _ptr(y))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    if debug:
        return rec, dict(g_pre=g_pre, s1_pre=s1_pre, z_pre=z_pre, y=y)
    return rec


def group_meta_given_s2(view: TileView, bits: int, axis: int, s2_bytes: np.ndarray, rotate: bool = True):
    """Pre-rounding s1 and zero-point when the FP8 second scale is s2_bytes [n][128]."""
    s2_bytes = np.ascontiguousarray(s2_bytes, np.uint8)
    s1_pre = np.empty((view.n, N), np.float64)
    z_pre = np.empty((view.n, N), np.float64)
    rc = lib().kvo_group_meta_given_s2(*view.args(), bits, axis, int(rotate), _ptr(s2_bytes), _ptr(s1_pre),
                                       _ptr(z_pre))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return s1_pre, z_pre


def codes_given_meta(view: TileView, bits: int, axis: int, records: np.ndarray, rotate: bool = True):
    """Codes [n][128][128] and unrounded t the oracle derives with the records' metadata."""
    records = np.ascontiguousarray(records, np.uint8)
    codes = np.empty((view.n, N, N), np.uint8)
    t = np.empty((view.n, N, N), np.float64)
    rc = lib().kvo_codes_given_meta(*view.args(), bits, axis, int(rotate), _ptr(records), _ptr(codes), _ptr(t))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return codes, t


def unpack_codes(records: np.ndarray, bits: int, axis: int) -> np.ndarray:
    """Codes of packed records as [n][128 tokens][128 channels] (code rows follow the s2 axis)."""
    records = np.ascontiguousarray(records, np.uint8).reshape(-1, record_bytes(bits))
    codes = np.empty((records.shape[0], N, N), np.uint8)
    if lib().kvo_unpack_codes(_ptr(records), records.shape[0], bits, axis, _ptr(codes)) != 0:
        raise ValueError("bad bits or axis")
    return codes


def dequantize(records: np.ndarray, bits: int, axis: int, rotate: bool = True) -> np.ndarray:
    records = np.ascontiguousarray(records, np.uint8).reshape(-1, record_bytes(bits))
    out = np.empty((records.shape[0], N, N), np.float64)
    if lib().kvo_dequantize_tiles(_ptr(records), records.shape[0], bits, axis, int(rotate), _ptr(out)) != 0:
        raise ValueError("oracle dequantize rejected its arguments")
    return out


def decode_attn(q_f16_bits, k_records, v_records, n_tiles, n_q_heads, n_kv_heads, max_tiles, bits_k, bits_v,
                sm_scale=None, block_table=None, rotate: bool = True, k_sink=None, v_sink=None, k_recent=None,
                v_recent=None, n_recent=None) -> np.ndarray:
    """out[b][hq][128] float64; q_f16_bits: uint16 [b][hq][128].  Optional FP16
    windows as uint16 bits: k_sink / v_sink [b][n_kv_heads][n_sink][128],
    k_recent / v_recent [b][n_kv_heads][recent_cap][128] with n_recent[b] valid."""
    q = np.ascontiguousarray(q_f16_bits, np.uint16)
    batch = q.shape[0]
    k = np.ascontiguousarray(k_records, np.uint8)
    v = np.ascontiguousarray(v_records, np.uint8)
    nt = np.ascontiguousarray(n_tiles, np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(N)
    ks = vs = kr = vr = nr = None
    n_sink = recent_cap = 0
    if k_sink is not None:
        ks, vs = np.ascontiguousarray(k_sink, np.uint16), np.ascontiguousarray(v_sink, np.uint16)
        n_sink = ks.shape[2]
    if k_recent is not None:
        kr, vr = np.ascontiguousarray(k_recent, np.uint16), np.ascontiguousarray(v_recent, np.uint16)
        nr = np.ascontiguousarray(n_recent, np.int32)
        recent_cap = kr.shape[2]
    out = np.empty((batch, n_q_heads, N), np.float64)
    rc = lib().kvo_decode_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(nt), batch, n_q_heads, n_kv_heads,
                               max_tiles, bits_k, bits_v, int(rotate), float(sm_scale), _ptr(ks), _ptr(vs), n_sink,
                               _ptr(kr), _ptr(vr), _ptr(nr), recent_cap, _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_attn rejected its arguments")
    return out


# --------------------------------------------------------------------------- record fields
def record_fields(records: np.ndarray, bits: int):
    """Split records [n][Pb] into (code bytes, s1 bytes, s2 bytes, z uint16)."""
    r = np.ascontiguousarray(records, np.uint8).reshape(-1, record_bytes(bits))
    c = 2048 * bits
    return (r[:, :c], r[:, c:c + 128], r[:, c + 128:c + 256],
            np.ascontiguousarray(r[:, c + 256:c + 512]).view(np.uint16))
