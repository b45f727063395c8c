"""Python binding of libkvarn.so (the C ABI in include/kvarn.h).

Argument marshalling only: every step of the codec runs in the HIP kernels of
``libkvarn.so``.  PyTorch supplies device memory (``Tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream()``).  There is no fallback: if the library
is missing, :func:`load` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvarn.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
F16, BF16, F32 = 0, 1, 2
AXIS_K, AXIS_V = 0, 1
NO_ROTATION = 1          # flag: the variant without the Walsh-Hadamard rotation (KIVI with n_iter = 0)
SINGLE_SCALE = 2         # read flag, with NO_ROTATION: KIVI records dequantised without a second scale
HEAD_DIM = TILE = 128

# Every function declared in include/kvarn.h, with its ctypes signature.
_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "kvarn_format_version": (_I, []),
    "kvarn_tile_bytes": (_SZ, [_I]),
    "kvarn_parse_preset": (_I, [ctypes.c_char_p, _P, _P, _P]),
    "kvarn_status_string": (ctypes.c_char_p, [_I]),
    "kvarn_quantize_tiles": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _P, _P, _I, _P]),
    "kvarn_dequantize_tiles": (_I, [_P, _P, _I64, _I, _I, _P, _I, _I64, _I64, _P, _I, _P]),
    "kvarn_decode_attn_workspace_bytes": (_SZ, [_I64, _I, _I, _I]),
    "kvarn_decode_attn": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _I, _P]),
    "kvarn_decode_attn_windows": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _I, _P, _P, _P,
                                       _I, _P, _P, _SZ, _I, _P]),
    "kvarn_decode_attn_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I, _I, _F, _P, _I, _P]),
}
NOALLOC_SCRATCH_BYTES = 16 << 20   # KVARN_NOALLOC_SCRATCH_BYTES

_lib = None


class KvarnError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libkvarn.so (built by ``python -m kv_cache_quantization_x128_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_quantization_x128_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().kvarn_status_string(int(status)).decode()


def tile_bytes(bits: int) -> int:
    return int(load().kvarn_tile_bytes(bits))


def format_version() -> int:
    return int(load().kvarn_format_version())


def parse_preset(preset: str):
    bk, bv, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = load().kvarn_parse_preset(preset.encode(), ctypes.byref(bk), ctypes.byref(bv), ctypes.byref(g))
    if st != OK:
        raise KvarnError("kvarn_parse_preset", st)
    return bk.value, bv.value, g.value


def workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_tiles: int) -> int:
    return int(load().kvarn_decode_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, max_tiles))


# --------------------------------------------------------------------------- helpers
_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}


def _ptr(t, dtype=None):
    """Device address of tensor t (None passes NULL).  The kernels dereference it
    on the GPU, so a host tensor is refused here; index tensors must also have
    the element type the C ABI reads."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkvarn takes device tensors; got one on " + str(t.device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected a {dtype} tensor, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


# Size checks on tensor metadata only (no device reads, no synchronisation): the
# kernels read and write the memory the arguments describe, so a tensor that is
# smaller than that, or not contiguous, is refused before the call instead of
# being read or written out of bounds on the GPU.  Index and offset values are
# the caller's to keep inside the buffers (the header says so).
def _nbytes(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.numel() * t.element_size()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_index(t, n, name, dtype):
    if t is not None:
        _need(t.dtype == dtype, f"{name}: expected {dtype}, got {t.dtype}")
        _need(_nbytes(t, name) >= n * t.element_size(), f"{name} has fewer than {n} entries")


def _check_tiles(buf, n_tiles, tile_stride, token_stride, offsets, name):
    """buf covers n_tiles tiles at these strides (or offsets has n_tiles entries)."""
    _check_index(offsets, n_tiles, name + " offsets", torch.int64)
    if offsets is None and n_tiles > 0 and tile_stride >= 0 and token_stride >= HEAD_DIM:
        last = (n_tiles - 1) * tile_stride + (TILE - 1) * token_stride + HEAD_DIM
        _need(_nbytes(buf, name) >= last * buf.element_size(),
              f"{name} holds fewer than {n_tiles} tiles at tile_stride {tile_stride}, token_stride {token_stride}")


def _check_records(buf, n_tiles, bits, index, name):
    """buf holds n_tiles records (or index has n_tiles entries)."""
    _check_index(index, n_tiles, name + " index", torch.int64)
    if index is None and n_tiles > 0:
        _need(_nbytes(buf, name) >= n_tiles * tile_bytes(bits), f"{name} holds fewer than {n_tiles} records")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != OK:
        raise KvarnError(fn, st)


# --------------------------------------------------------------------------- entry points
def quantize_tiles(x: torch.Tensor, n_tiles: int, bits: int, axis: int, *, tile_stride: int = TILE * HEAD_DIM,
                   token_stride: int = HEAD_DIM, tile_offset: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, dst_index: torch.Tensor | None = None, n_iter: int = 8,
                   flags: int = 0, stream=None) -> torch.Tensor:
    """Quantise tiles of ``x`` (fp16/bf16/fp32 on the GPU) into packed uint8 records [n, Pb]."""
    if out is None:
        out = torch.empty((n_tiles, tile_bytes(bits)), dtype=torch.uint8, device=x.device)
    _check_tiles(x, n_tiles, tile_stride, token_stride, tile_offset, "x")
    _check_records(out, n_tiles, bits, dst_index, "out")
    st = load().kvarn_quantize_tiles(_ptr(x), _DT[x.dtype], n_tiles, tile_stride, token_stride,
                                     _ptr(tile_offset, torch.int64), bits, axis, n_iter, _ptr(out),
                                     _ptr(dst_index, torch.int64), flags, _stream(stream))
    _check("kvarn_quantize_tiles", st)
    return out


def quantize(x: torch.Tensor, bits: int, axis: int, n_iter: int = 8, flags: int = 0, stream=None) -> torch.Tensor:
    """Dense ``x[..., T, 128]`` (T a multiple of 128, contiguous) -> records [x.numel() / 16384, Pb]."""
    assert x.is_contiguous() and x.shape[-1] == HEAD_DIM and x.shape[-2] % TILE == 0
    return quantize_tiles(x, x.numel() // (TILE * HEAD_DIM), bits, axis, n_iter=n_iter, flags=flags, stream=stream)


def dequantize_tiles(packed: torch.Tensor, n_tiles: int, bits: int, axis: int, out: torch.Tensor, *,
                     tile_stride: int = TILE * HEAD_DIM, token_stride: int = HEAD_DIM,
                     src_index: torch.Tensor | None = None, dst_offset: torch.Tensor | None = None,
                     flags: int = 0, stream=None) -> torch.Tensor:
    _check_records(packed, n_tiles, bits, src_index, "packed")
    _check_tiles(out, n_tiles, tile_stride, token_stride, dst_offset, "out")
    st = load().kvarn_dequantize_tiles(_ptr(packed), _ptr(src_index, torch.int64), n_tiles, bits, axis,
                                       _ptr(out), _DT[out.dtype], tile_stride, token_stride,
                                       _ptr(dst_offset, torch.int64), flags,
                                       _stream(stream))
    _check("kvarn_dequantize_tiles", st)
    return out


def dequantize(packed: torch.Tensor, bits: int, axis: int, dtype=torch.float32, flags: int = 0,
               stream=None) -> torch.Tensor:
    """Records [n, Pb] -> tiles [n, 128, 128] of ``dtype``."""
    n = packed.shape[0]
    out = torch.empty((n, TILE, HEAD_DIM), dtype=dtype, device=packed.device)
    return dequantize_tiles(packed, n, bits, axis, out, flags=flags, stream=stream)


def decode_attn(q: torch.Tensor, k_packed: torch.Tensor, v_packed: torch.Tensor, n_tiles_per_seq: torch.Tensor,
                n_kv_heads: int, max_tiles: int, bits_k: int, bits_v: int, *, block_table: torch.Tensor | None = None,
                sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, flags: int = 0, k_sink: torch.Tensor | None = None,
                v_sink: torch.Tensor | None = None, k_recent: torch.Tensor | None = None,
                v_recent: torch.Tensor | None = None, n_recent: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """q fp16 [batch][n_q_heads][128] -> attention output fp16 of the same shape.

    Optional FP16 windows around the packed body: k_sink / v_sink
    [batch][n_kv_heads][n_sink][128]; k_recent / v_recent
    [batch][n_kv_heads][recent_cap][128] with n_recent int32 [batch] valid tokens."""
    _need(q.dim() == 3 and q.shape[2] == HEAD_DIM and q.dtype == torch.float16, "q: fp16 [batch][n_q_heads][128]")
    batch, n_q_heads, _ = q.shape
    _nbytes(q, "q")
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == torch.float16 and out.is_contiguous(), "out: contiguous, like q")
    need = workspace_bytes(batch, n_q_heads, n_kv_heads, max_tiles)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _nbytes(workspace, "workspace")
    _check_index(n_tiles_per_seq, batch, "n_tiles_per_seq", torch.int32)
    _check_index(block_table, batch * n_kv_heads * max(max_tiles, 0), "block_table", torch.int32)
    # records past the end of either buffer count as missing tiles in the kernel
    tbk, tbv = tile_bytes(bits_k), tile_bytes(bits_v)
    n_records = min(_nbytes(k_packed, "k_packed") // tbk, _nbytes(v_packed, "v_packed") // tbv) if tbk and tbv else 0
    for kw, vw, name in ((k_sink, v_sink, "sink"), (k_recent, v_recent, "recent")):
        if kw is not None or vw is not None:
            _need(kw is not None and vw is not None and kw.shape == vw.shape, f"k_{name} and v_{name} go together")
            _need(kw.dim() == 4 and tuple(kw.shape[:2]) == (batch, n_kv_heads) and kw.shape[3] == HEAD_DIM and
                  kw.dtype == torch.float16 and vw.dtype == torch.float16,
                  f"{name} windows: fp16 [batch][n_kv_heads][n][128]")
            _nbytes(kw, "k_" + name), _nbytes(vw, "v_" + name)
    if k_recent is not None:
        _need(n_recent is not None, "n_recent goes with the recent windows")
        _check_index(n_recent, batch, "n_recent", torch.int32)
    if k_sink is None and k_recent is None:
        st = load().kvarn_decode_attn(_ptr(q), _ptr(k_packed), _ptr(v_packed), _ptr(block_table, torch.int32),
                                      _ptr(n_tiles_per_seq, torch.int32), n_records, batch, n_q_heads, n_kv_heads,
                                      max_tiles, bits_k, bits_v, float(sm_scale), _ptr(out), _ptr(workspace),
                                      ws_bytes, flags, _stream(stream))
        _check("kvarn_decode_attn", st)
        return out
    n_sink = 0 if k_sink is None else k_sink.shape[2]
    cap = 0 if k_recent is None else k_recent.shape[2]
    st = load().kvarn_decode_attn_windows(_ptr(q), _ptr(k_packed), _ptr(v_packed), _ptr(block_table, torch.int32),
                                          _ptr(n_tiles_per_seq, torch.int32), n_records, batch, n_q_heads,
                                          n_kv_heads, max_tiles, bits_k, bits_v, float(sm_scale), _ptr(k_sink),
                                          _ptr(v_sink), n_sink,
                                          _ptr(k_recent), _ptr(v_recent), _ptr(n_recent, torch.int32), cap, _ptr(out),
                                          _ptr(workspace), ws_bytes, flags, _stream(stream))
    _check("kvarn_decode_attn_windows", st)
    return out


def decode_attn_noalloc(q: torch.Tensor, k_packed: torch.Tensor, v_packed: torch.Tensor,
                        n_tiles_per_seq: torch.Tensor, n_kv_heads: int, max_tiles: int, bits_k: int, bits_v: int, *,
                        out: torch.Tensor, block_table: torch.Tensor | None = None, sm_scale: float | None = None,
                        flags: int = 0, stream=None) -> torch.Tensor:
    """kvarn_decode_attn_noalloc: decode attention with the library's device
    scratch in place of a workspace.  ``out`` (fp16, like q) is the caller's; the
    call allocates nothing, here or in the library."""
    _need(q.dim() == 3 and q.shape[2] == HEAD_DIM and q.dtype == torch.float16, "q: fp16 [batch][n_q_heads][128]")
    batch, n_q_heads, _ = q.shape
    _nbytes(q, "q")
    _need(out.shape == q.shape and out.dtype == torch.float16 and out.is_contiguous(), "out: contiguous, like q")
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    _check_index(n_tiles_per_seq, batch, "n_tiles_per_seq", torch.int32)
    _check_index(block_table, batch * n_kv_heads * max(max_tiles, 0), "block_table", torch.int32)
    tbk, tbv = tile_bytes(bits_k), tile_bytes(bits_v)
    n_records = min(_nbytes(k_packed, "k_packed") // tbk, _nbytes(v_packed, "v_packed") // tbv) if tbk and tbv else 0
    st = load().kvarn_decode_attn_noalloc(_ptr(q), _ptr(k_packed), _ptr(v_packed), _ptr(block_table, torch.int32),
                                          _ptr(n_tiles_per_seq, torch.int32), n_records, batch, n_q_heads, n_kv_heads,
                                          max_tiles, bits_k, bits_v, float(sm_scale), _ptr(out), flags,
                                          _stream(stream))
    _check("kvarn_decode_attn_noalloc", st)
    return out
