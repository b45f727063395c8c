"""The seeded generators are deterministic and produce the documented shapes and outlier structure."""
import numpy as np
import torch

from kv_cache_quantization_x128_amd import synth


def test_tiny_shape_and_determinism():
    k1, v1 = synth.tiny()
    k2, v2 = synth.tiny()
    assert k1.shape == (1, 1, 1024, 128) and k1.dtype == np.float16
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.array_equal(k1, v1)
    # four outlier channels x15: their RMS stands out
    rms = np.sqrt((k1[0, 0].astype(np.float64) ** 2).mean(0))
    assert (rms > 8).sum() == 4


def test_small_decode_append_layout_cpu():
    k, v = synth.decode_append(n_layers=2, n_seq=3, n_heads=2, device="cpu")
    assert k.shape == (2, 3, 128, 2, 128) and k.dtype == torch.bfloat16
    k2, _ = synth.decode_append(n_layers=2, n_seq=3, n_heads=2, device="cpu")
    assert torch.equal(k, k2)
    off = synth.decode_append_offsets(2, 3, 2, device="cpu")
    flat = k.reshape(-1)
    # tile (layer 1, seq 2, head 1), token 5, channel 7
    t = (1 * 3 + 2) * 2 + 1
    assert flat[off[t] + 5 * 2 * 128 + 7] == k[1, 2, 5, 1, 7]


def test_decode_attn_layer_plants_peaked_keys_cpu():
    g = synth.generator(1005, "cpu")
    q, k, v = synth.decode_attn_layer(g, n_seq=2, n_kv_heads=2, n_q_heads=8, n_tokens=512, device="cpu")
    assert q.shape == (2, 8, 128) and k.shape == (2, 2, 512, 128)
    kk = k.float().repeat_interleave(4, dim=1)                      # [seq][8 q heads][tok][128]
    logits = torch.matmul(kk, q.float()[..., None])[..., 0] / np.sqrt(128)
    top = logits.topk(8, dim=-1).values.mean(-1)
    assert (top > 6).all()
