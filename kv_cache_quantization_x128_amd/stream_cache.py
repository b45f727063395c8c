"""A streaming KV cache around the codec: FP16 sink, packed body, FP16 trailing window.

The pages keep the first S = 128 tokens of every sequence and its most recent
tokens (up to R = 128) in FP16 and quantise the 128-token blocks in between
(paperlayer.ai summary, appendix D); a block is quantised when it fills
(pheeree.github.io blog, part 3).  This class only does the bookkeeping around
the C ABI: device buffers come from PyTorch, every block fill is one
``kvarn_quantize_tiles`` call per K and V for all the (sequence, KV head) pairs
that filled, reading the tiles in place from the trailing-window buffer and
writing the records into the next free slots of a shared record pool, and
attention is one ``kvarn_decode_attn_windows`` call.

Layout (all device tensors):
  sink_k, sink_v       fp16 [batch][n_kv_heads][S][128]
  recent_k, recent_v   fp16 [batch][n_kv_heads][R][128]
  pool_k, pool_v       uint8 [batch * n_kv_heads * max_tiles][record bytes]
  block_table          int32 [batch * n_kv_heads * max_tiles]: record of tile j of
                       (b, h) at row (b * n_kv_heads + h) * max_tiles + j
  n_tiles, n_recent    int32 [batch]
"""
from __future__ import annotations

import torch

from . import kvarn

TILE = kvarn.TILE


class StreamingKVCache:
    def __init__(self, batch: int, n_kv_heads: int, max_tiles: int, bits_k: int = 2, bits_v: int = 2,
                 n_sink: int = 128, recent_cap: int = TILE, flags: int = 0, n_iter: int = 8, device="cuda"):
        if recent_cap != TILE:
            raise ValueError("the trailing window holds exactly one block (128 tokens) before it is quantised")
        if n_sink < 0 or batch <= 0 or n_kv_heads <= 0 or max_tiles <= 0:
            raise ValueError("bad cache shape")
        self.batch, self.n_kv_heads, self.max_tiles = batch, n_kv_heads, max_tiles
        self.bits_k, self.bits_v, self.n_sink, self.cap, self.flags = bits_k, bits_v, n_sink, recent_cap, flags
        self.n_iter = n_iter   # normalisation rounds (0 with KVARN_NO_ROTATION: the KIVI records)
        dev = torch.device(device)
        f16 = dict(dtype=torch.float16, device=dev)
        self.sink_k = torch.zeros((batch, n_kv_heads, max(n_sink, 1), 128), **f16)
        self.sink_v = torch.zeros_like(self.sink_k)
        self.recent_k = torch.zeros((batch, n_kv_heads, recent_cap, 128), **f16)
        self.recent_v = torch.zeros_like(self.recent_k)
        rows = batch * n_kv_heads * max_tiles
        self.pool_k = torch.zeros((rows, kvarn.tile_bytes(bits_k)), dtype=torch.uint8, device=dev)
        self.pool_v = torch.zeros((rows, kvarn.tile_bytes(bits_v)), dtype=torch.uint8, device=dev)
        self.block_table = torch.full((rows,), -1, dtype=torch.int32, device=dev)
        self.n_tiles = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.n_recent = torch.zeros(batch, dtype=torch.int32, device=dev)
        # host mirrors of the counts (the caller's appends are known on the host)
        self._tiles = [0] * batch
        self._recent = [0] * batch
        self._prefilled = False
        self._next_record = 0
        self._heads = torch.arange(n_kv_heads, device=dev, dtype=torch.int64)

    # ------------------------------------------------------------------ filling
    def prefill(self, k: torch.Tensor, v: torch.Tensor, lengths=None) -> None:
        """Prompt tokens k, v fp16 [batch][n_kv_heads][T][128]; sequence b uses its
        first lengths[b] (default T) tokens, at least the sink's S.  The sink takes
        the first S, every full block after it is quantised into the body and the
        rest starts the trailing window."""
        if self._prefilled:
            raise RuntimeError("prefill() is called once, before append()")
        self._check_tokens(k, v, 4)
        T = k.shape[2]
        lengths = [T] * self.batch if lengths is None else [int(x) for x in lengths]
        if len(lengths) != self.batch:
            raise ValueError("one length per sequence")
        if any(L < self.n_sink or L > T for L in lengths):
            raise ValueError("every sequence needs at least the sink's tokens, and at most T")
        if any((L - self.n_sink) // TILE > self.max_tiles for L in lengths):
            raise ValueError("prompt longer than the cache's capacity")
        if self.n_sink:
            self.sink_k.copy_(k[:, :, :self.n_sink])
            self.sink_v.copy_(v[:, :, :self.n_sink])
        for b, L in enumerate(lengths):
            n_blocks = (L - self.n_sink) // TILE
            for j in range(n_blocks):
                t0 = self.n_sink + j * TILE
                self.recent_k[b].copy_(k[b, :, t0:t0 + TILE])
                self.recent_v[b].copy_(v[b, :, t0:t0 + TILE])
                self._commit([b])
            r = L - self.n_sink - n_blocks * TILE
            if r:
                t0 = self.n_sink + n_blocks * TILE
                self.recent_k[b, :, :r].copy_(k[b, :, t0:t0 + r])
                self.recent_v[b, :, :r].copy_(v[b, :, t0:t0 + r])
            self._recent[b] = r
        self.n_recent.copy_(torch.tensor(self._recent, dtype=torch.int32))
        self._prefilled = True

    def append(self, k: torch.Tensor, v: torch.Tensor, active=None) -> None:
        """One new token per sequence: k, v fp16 [batch][n_kv_heads][128].  Rows of
        sequences not in `active` (default: all) are ignored.  Sequences whose
        trailing window fills get that block quantised into the body."""
        if not self._prefilled:
            raise RuntimeError("prefill() first (the sink needs its tokens)")
        self._check_tokens(k, v, 3)
        seqs = list(range(self.batch)) if active is None else [int(b) for b in active]
        if len(set(seqs)) != len(seqs) or any(b < 0 or b >= self.batch for b in seqs):
            raise ValueError("active sequences must be distinct indices below batch")
        if not seqs:
            return
        # every check before the first write: a refused call leaves the cache as it was
        full = [b for b in seqs if self._recent[b] + 1 == self.cap]
        if any(self._tiles[b] >= self.max_tiles for b in full):
            raise RuntimeError("a sequence outgrew the cache's capacity")
        idx = torch.tensor(seqs, device=k.device, dtype=torch.int64)
        pos = torch.tensor([self._recent[b] for b in seqs], device=k.device, dtype=torch.int64)
        self.recent_k[idx, :, pos] = k[idx]
        self.recent_v[idx, :, pos] = v[idx]
        for b in seqs:
            self._recent[b] += 1
        if full:
            self._commit(full)
            for b in full:
                self._recent[b] = 0
        self.n_recent.copy_(torch.tensor(self._recent, dtype=torch.int32))

    def _check_tokens(self, k: torch.Tensor, v: torch.Tensor, ndim: int) -> None:
        """k and v: fp16 on the cache's device, [batch][n_kv_heads][T][128] (ndim 4,
        prefill) or [batch][n_kv_heads][128] (ndim 3, append)."""
        for t in (k, v):
            if (t.dtype != torch.float16 or t.device != self.recent_k.device or t.dim() != ndim or
                    t.shape[:2] != (self.batch, self.n_kv_heads) or t.shape[-1] != 128):
                raise ValueError(f"expected fp16 [{self.batch}][{self.n_kv_heads}]{'[T]' if ndim == 4 else ''}[128] "
                                 f"on {self.recent_k.device}, got {t.dtype} {tuple(t.shape)} on {t.device}")
        if k.shape != v.shape:
            raise ValueError("k and v differ in shape")

    def _commit(self, seqs) -> None:
        """Quantise the full trailing windows of `seqs` (all their KV heads) into
        the next free records and enter them in the block table."""
        h = self.n_kv_heads
        b = torch.tensor(seqs, device=self.recent_k.device, dtype=torch.int64)
        offs = ((b[:, None] * h + self._heads[None, :]) * (self.cap * 128)).reshape(-1)
        n = offs.numel()
        dst = torch.arange(self._next_record, self._next_record + n, device=offs.device, dtype=torch.int64)
        kvarn.quantize_tiles(self.recent_k, n, self.bits_k, kvarn.AXIS_K, tile_offset=offs, out=self.pool_k,
                             dst_index=dst, n_iter=self.n_iter, flags=self.flags)
        kvarn.quantize_tiles(self.recent_v, n, self.bits_v, kvarn.AXIS_V, tile_offset=offs, out=self.pool_v,
                             dst_index=dst, n_iter=self.n_iter, flags=self.flags)
        rows = torch.tensor([(bb * h + hh) * self.max_tiles + self._tiles[bb] for bb in seqs for hh in range(h)],
                            device=offs.device, dtype=torch.int64)
        self.block_table[rows] = dst.to(torch.int32)
        self._next_record += n
        for bb in seqs:
            self._tiles[bb] += 1
        self.n_tiles.copy_(torch.tensor(self._tiles, dtype=torch.int32))

    # ------------------------------------------------------------------ reading
    def attend(self, q: torch.Tensor, sm_scale: float | None = None, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
        """Decode attention of q fp16 [batch][n_q_heads][128] over sink + body +
        trailing window."""
        return kvarn.decode_attn(q, self.pool_k, self.pool_v, self.n_tiles, self.n_kv_heads, self.max_tiles,
                                 self.bits_k, self.bits_v, block_table=self.block_table, sm_scale=sm_scale, out=out,
                                 workspace=workspace, flags=self.flags,
                                 k_sink=self.sink_k if self.n_sink else None,
                                 v_sink=self.sink_v if self.n_sink else None,
                                 k_recent=self.recent_k, v_recent=self.recent_v, n_recent=self.n_recent)

    def tokens(self, b: int) -> int:
        """Tokens held for sequence b."""
        return self.n_sink + TILE * self._tiles[b] + self._recent[b]
