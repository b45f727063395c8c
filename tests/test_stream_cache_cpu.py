"""Host-side checks of the streaming cache: every misuse is refused before any
write or library call, so these run on a machine without a GPU (the cache's
buffers live on the CPU here and no block ever fills)."""
import pytest
import torch

from kv_cache_quantization_x128_amd.stream_cache import StreamingKVCache


def _cache(**kw):
    args = dict(batch=2, n_kv_heads=2, max_tiles=1, device="cpu")
    args.update(kw)
    return StreamingKVCache(**args)


def _tok(*shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def test_construction_checks():
    with pytest.raises(ValueError):
        _cache(recent_cap=64)
    with pytest.raises(ValueError):
        _cache(batch=0)
    with pytest.raises(ValueError):
        _cache(max_tiles=0)


def test_prefill_checks():
    c = _cache()
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 200, 128, dtype=torch.bfloat16), _tok(2, 2, 200, 128))   # not fp16
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 3, 200, 128), _tok(2, 3, 200, 128))                          # wrong head count
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 200, 128), _tok(2, 2, 199, 128))                          # k and v differ
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 200, 128), _tok(2, 2, 200, 128), lengths=[200])           # one length per sequence
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 200, 128), _tok(2, 2, 200, 128), lengths=[200, 100])      # shorter than the sink
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 200, 128), _tok(2, 2, 200, 128), lengths=[200, 201])      # longer than T
    with pytest.raises(ValueError):
        c.prefill(_tok(2, 2, 512, 128), _tok(2, 2, 512, 128))                          # two blocks, room for one
    with pytest.raises(RuntimeError):
        c.append(_tok(2, 2, 128), _tok(2, 2, 128))                                     # before prefill


def test_prefill_without_blocks_and_append_checks():
    c = _cache()
    k = torch.arange(2 * 2 * 200 * 128, dtype=torch.float32).reshape(2, 2, 200, 128).half()
    c.prefill(k, k, lengths=[130, 200])          # sink plus partial windows only: nothing is quantised
    assert [c.tokens(b) for b in range(2)] == [130, 200]
    assert c.n_recent.tolist() == [2, 72] and c.n_tiles.tolist() == [0, 0]
    assert torch.equal(c.sink_k, k[:, :, :128]) and torch.equal(c.recent_k[1, :, :72], k[1, :, 128:200])
    with pytest.raises(RuntimeError):
        c.prefill(k, k)                          # once only
    t = _tok(2, 2, 128)
    for bad in ([0, 0], [2], [-1]):
        with pytest.raises(ValueError):
            c.append(t, t, active=bad)
    with pytest.raises(ValueError):
        c.append(_tok(2, 2, 64), _tok(2, 2, 64))
    assert [c.tokens(b) for b in range(2)] == [130, 200]    # refused calls changed nothing
    c.append(t + 1, t + 2, active=[1])
    assert [c.tokens(b) for b in range(2)] == [130, 201] and c.n_recent.tolist() == [2, 73]
    assert bool((c.recent_k[1, :, 72] == 1).all()) and bool((c.recent_v[1, :, 72] == 2).all())
    c.append(t, t, active=[])
    assert [c.tokens(b) for b in range(2)] == [130, 201]
