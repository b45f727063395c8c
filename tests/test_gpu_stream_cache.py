"""The streaming cache (FP16 sink, packed body, FP16 trailing window) built on
the C ABI: block fills land in the record pool exactly as a direct quantisation
of the same tokens, and decode attention over the three regions matches the
oracle at every fill."""
import numpy as np
import pytest
import torch

import oracle
import parity
from kv_cache_quantization_x128_amd import kvarn
from kv_cache_quantization_x128_amd.stream_cache import StreamingKVCache

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _log(*a):
    print(*a, flush=True)


def _oracle_pools(c, hist_k, hist_v, n_sink=128):
    """The record pools as the oracle writes them from the tokens each sequence
    received (hist_*[b]: fp16 [n_kv_heads][tokens][128] in arrival order): tile j
    of (b, h) is tokens n_sink + 128 j ... at the record the block table names."""
    pk = np.zeros(tuple(c.pool_k.shape), np.uint8)
    pv = np.zeros(tuple(c.pool_v.shape), np.uint8)
    tab, nts = c.block_table.cpu().numpy(), c.n_tiles.cpu().numpy()
    for b in range(len(hist_k)):
        for h in range(c.n_kv_heads):
            for j in range(int(nts[b])):
                r = int(tab[(b * c.n_kv_heads + h) * c.max_tiles + j])
                t0 = n_sink + 128 * j
                for pool, hist, axis, bits in ((pk, hist_k, kvarn.AXIS_K, c.bits_k), (pv, hist_v, kvarn.AXIS_V, c.bits_v)):
                    x = np.ascontiguousarray(hist[b][h, t0:t0 + 128]).view(np.uint16)
                    pool[r] = oracle.quantize(oracle.TileView.dense(x, oracle.DT_F16), bits, axis,
                                              n_iter=c.n_iter, rotate=not c.flags)[0]
    return pk, pv


def _oracle_attend(c, q, hist_k, hist_v):
    u16 = lambda t: t.contiguous().cpu().numpy().view(np.uint16)  # noqa: E731
    hq = q.shape[1]
    pk, pv = _oracle_pools(c, hist_k, hist_v)
    return oracle.decode_attn(u16(q), pk, pv, c.n_tiles.cpu().numpy(), hq,
                              c.n_kv_heads, c.max_tiles, c.bits_k, c.bits_v, block_table=c.block_table.cpu().numpy(),
                              rotate=not c.flags, k_sink=u16(c.sink_k), v_sink=u16(c.sink_v), k_recent=u16(c.recent_k),
                              v_recent=u16(c.recent_v), n_recent=c.n_recent.cpu().numpy())


@pytest.mark.parametrize("bits_k,bits_v,flags,n_iter", [(2, 2, 0, 8), (4, 2, 0, 8), (2, 2, kvarn.NO_ROTATION, 0)])
def test_stream_cache_prefill_append_attend(dev, bits_k, bits_v, flags, n_iter):
    batch, hkv, gs, max_tiles = 3, 2, 4, 5
    hq = hkv * gs
    g = torch.Generator(device=dev).manual_seed(123 + bits_k)
    T = 128 + 5 * 128
    k = (torch.randn((batch, hkv, T, 128), generator=g, device=dev) *
         torch.exp(0.5 * torch.randn((1, hkv, 1, 128), generator=g, device=dev))).half()
    v = torch.randn((batch, hkv, T, 128), generator=g, device=dev).half()
    q = torch.randn((batch, hq, 128), generator=g, device=dev).half()
    c = StreamingKVCache(batch, hkv, max_tiles, bits_k, bits_v, flags=flags, n_iter=n_iter, device=dev)
    prompt = [128 + 2 * 128 + 30, 128 + 77, 128 + 128]
    c.prefill(k, v, lengths=prompt)
    assert [c.tokens(b) for b in range(batch)] == prompt
    assert c.n_tiles.tolist() == [2, 0, 1] and c.n_recent.tolist() == [30, 77, 0]
    # the body holds exactly what a direct quantisation of the same block gives
    direct = kvarn.quantize(k[0, :, 128 + 128:128 + 256].contiguous(), bits_k, kvarn.AXIS_K, n_iter=n_iter,
                            flags=flags)
    rows = [(0 * hkv + h) * max_tiles + 1 for h in range(hkv)]
    rec = c.block_table[rows].long()
    assert torch.equal(c.pool_k[rec], direct)
    pos = list(prompt)
    hist_k = [k[b, :, :prompt[b]].cpu().numpy() for b in range(batch)]     # tokens received, per sequence
    hist_v = [v[b, :, :prompt[b]].cpu().numpy() for b in range(batch)]
    fills = 0
    for step in range(180):
        active = [b for b in range(batch) if not (b == 1 and step % 3 == 0)]   # sequence 1 skips some steps
        tiles_before = c.n_tiles.tolist()
        kt = torch.stack([k[b, :, min(pos[b], T - 1)] for b in range(batch)])
        vt = torch.stack([v[b, :, min(pos[b], T - 1)] for b in range(batch)])
        c.append(kt, vt, active=active)
        for b in active:
            pos[b] += 1
            hist_k[b] = np.concatenate([hist_k[b], kt[b].cpu().numpy()[:, None]], axis=1)
            hist_v[b] = np.concatenate([hist_v[b], vt[b].cpu().numpy()[:, None]], axis=1)
        if c.n_tiles.tolist() != tiles_before or step == 179:
            fills += c.n_tiles.tolist() != tiles_before
            got = c.attend(q).float().cpu().numpy()
            torch.cuda.synchronize()
            err = parity.rel_l2_rows(got, _oracle_attend(c, q, hist_k, hist_v))
            _log("stream cache", bits_k, bits_v, "step", step, "tiles", c.n_tiles.tolist(), "recent",
                 c.n_recent.tolist(), "max rel l2", err.max())
            assert err.max() <= TOL
    assert fills >= 2
    assert [c.tokens(b) for b in range(batch)] == pos


def test_stream_cache_rejects_misuse(dev):
    c = StreamingKVCache(1, 1, 1, device=dev)
    x = torch.zeros((1, 1, 64, 128), dtype=torch.float16, device=dev)
    with pytest.raises(RuntimeError):
        c.append(x[:, :, 0], x[:, :, 0])             # before prefill
    with pytest.raises(ValueError):
        c.prefill(x, x)                               # fewer tokens than the sink
    y = torch.zeros((1, 1, 128 + 128 + 127, 128), dtype=torch.float16, device=dev)
    c.prefill(y, y)
    for _ in range(2):                                # refused calls leave the cache as it was
        with pytest.raises(RuntimeError):
            c.append(y[:, :, 0], y[:, :, 0])         # the window fills but the body is full
        assert c.tokens(0) == 128 + 128 + 127 and c.n_recent.tolist() == [127]
