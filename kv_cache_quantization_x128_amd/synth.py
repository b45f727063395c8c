"""Seeded synthetic K/V inputs shaped like the workloads the KVarN pages evaluate.

This module generates data only; it contains none of the codec's arithmetic and
is the one piece shared by the tests, the benchmark and the oracle checks.

The pages measure on Qwen3-4B (36 layers, 8 KV heads, head_dim 128) and
Phi-4-14B (40 layers, 10 KV heads) KV caches (paperlayer.ai summary of arXiv
2606.03458v1, section 4 Experiments and appendix D).  No model weights or
datasets exist here, so these tensors stand in for them:

* values are N(0, 1);
* a few channels per (layer, KV head) are outlier channels, scaled up;
* each token is, with probability 5 %, an outlier token, scaled x4;
* keys get a RoPE-like rotation of the channel pairs (j, j + 64) with angle
  pos * 1e6 ** (-j / 64) -- the base 1e6 is this generator's choice;
* everything is rounded to the storage dtype (fp16 or bf16) at the end.

Workloads (seed, shape, storage order):

=================  =====  ===========================================  ===============
name               seed   shape                                        order
=================  =====  ===========================================  ===============
tiny               1001   K, V [1 layer][1 head][1024 tok][128] fp16   dense tiles
decode_append      1002   K, V [36][64 seq][128 tok][8 heads][128] bf16 token-major heads
prefill            1003   K, V [36][8 heads][32768 tok][128] bf16       dense tiles
phi4               1004   K, V [40][10 heads][8 seq][16384 tok][128]    dense tiles
decode_attn        1005   caches [16 seq][8 kv][32768 tok][128], q [16][32][128] fp16
=================  =====  ===========================================  ===============

``tiny`` is drawn with numpy's PCG64 on the host; the others are drawn with a
seeded ``torch.Generator`` on whichever device the caller names, so a GPU run
and a later host check read the very same bytes (the host copies them back).
"""
from __future__ import annotations

import math

import numpy as np
import torch

HEAD_DIM = 128
TILE = 128
ROPE_BASE = 1.0e6


# --------------------------------------------------------------------------- tiny (host)
def tiny(seed: int = 1001, n_tokens: int = 1024):
    """K and V, each float16 numpy [1][1][n_tokens][128]: N(0,1), 4 channels x15, 5 % tokens x4."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(2):
        x = rng.standard_normal((n_tokens, HEAD_DIM))
        ch = rng.choice(HEAD_DIM, size=4, replace=False)
        x[:, ch] *= 15.0
        tok = rng.random(n_tokens) < 0.05
        x[tok, :] *= 4.0
        out.append(x.astype(np.float16).reshape(1, 1, n_tokens, HEAD_DIM))
    return out[0], out[1]


# --------------------------------------------------------------------------- generic (torch)
def _rope(x: torch.Tensor, pos: torch.Tensor) -> torch.Tensor:
    """Rotate channel pairs (j, j+64) of x[..., T, 128] by angle pos[..., T] * base^(-j/64)."""
    half = HEAD_DIM // 2
    j = torch.arange(half, device=x.device, dtype=torch.float64)
    inv = ROPE_BASE ** (-j / half)
    ang = pos.to(torch.float64)[..., None] * inv
    cos, sin = torch.cos(ang).to(x.dtype), torch.sin(ang).to(x.dtype)
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1)


def outlier_heads(gen: torch.Generator, n_heads: int, n_seq: int, n_tokens: int, *, n_out_ch: int,
                  ch_scale: float, tok_p: float = 0.05, tok_scale: float = 4.0, rope_pos=None,
                  device="cpu") -> torch.Tensor:
    """One layer of K or V as float32 [n_heads][n_seq][n_tokens][128].

    Outlier channels are drawn once per head; outlier tokens independently per
    (head, sequence, token).  ``rope_pos`` ([n_seq][n_tokens] positions) turns on
    the key rotation.
    """
    x = torch.randn((n_heads, n_seq, n_tokens, HEAD_DIM), generator=gen, device=device, dtype=torch.float32)
    scores = torch.rand((n_heads, HEAD_DIM), generator=gen, device=device)
    ch = torch.argsort(scores, dim=1)[:, :n_out_ch]
    chs = torch.ones((n_heads, HEAD_DIM), device=device)
    chs.scatter_(1, ch, ch_scale)
    x *= chs[:, None, None, :]
    tok = torch.rand((n_heads, n_seq, n_tokens), generator=gen, device=device) < tok_p
    x *= torch.where(tok, tok_scale, 1.0)[..., None]
    if rope_pos is not None:
        x = _rope(x, rope_pos[None].to(device))
    return x


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------- workloads
def decode_append(seed: int = 1002, n_layers: int = 36, n_seq: int = 64, n_heads: int = 8, device="cuda",
                  dtype=torch.bfloat16):
    """K, V [L][n_seq][128 tokens][n_heads][128]: one new 128-token block per sequence.

    Outlier model of the tiny case (4 channels x15 per (layer, head), 5 % tokens
    x4).  Keys are rotated at positions start_b + t with start_b = 128 * U{0..255}.
    """
    g = _gen(seed, device)
    start = 128 * torch.randint(0, 256, (n_seq,), generator=g, device=device)
    pos = start[:, None] + torch.arange(TILE, device=device)[None, :]
    k = torch.empty((n_layers, n_seq, TILE, n_heads, HEAD_DIM), device=device, dtype=dtype)
    v = torch.empty_like(k)
    for layer in range(n_layers):
        for dst, rp in ((k, pos), (v, None)):
            x = outlier_heads(g, n_heads, n_seq, TILE, n_out_ch=4, ch_scale=15.0, rope_pos=rp, device=device)
            dst[layer] = x.permute(1, 2, 0, 3).to(dtype)
    return k, v


def decode_append_offsets(n_layers: int, n_seq: int, n_heads: int, device="cuda") -> torch.Tensor:
    """Element offset of tile (layer, seq, head) in the decode_append layout, in that order."""
    l = torch.arange(n_layers, device=device, dtype=torch.int64)[:, None, None]
    b = torch.arange(n_seq, device=device, dtype=torch.int64)[None, :, None]
    h = torch.arange(n_heads, device=device, dtype=torch.int64)[None, None, :]
    off = ((l * n_seq + b) * TILE * n_heads + h) * HEAD_DIM
    return off.reshape(-1).contiguous()


def prefill(seed: int = 1003, n_layers: int = 36, n_heads: int = 8, n_tokens: int = 32768, device="cuda",
            dtype=torch.bfloat16):
    """K, V [L][n_heads][n_tokens][128]: 3 outlier channels (2 % of 128) x20, 5 % tokens x4, keys rotated."""
    g = _gen(seed, device)
    pos = torch.arange(n_tokens, device=device)[None, :]
    k = torch.empty((n_layers, n_heads, n_tokens, HEAD_DIM), device=device, dtype=dtype)
    v = torch.empty_like(k)
    for layer in range(n_layers):
        for dst, rp in ((k, pos), (v, None)):
            x = outlier_heads(g, n_heads, 1, n_tokens, n_out_ch=3, ch_scale=20.0, rope_pos=rp, device=device)
            dst[layer] = x[:, 0].to(dtype)
    return k, v


def phi4(seed: int = 1004, n_layers: int = 40, n_heads: int = 10, n_seq: int = 8, n_tokens: int = 16384,
         device="cuda", dtype=torch.bfloat16):
    """K, V [L][n_heads][n_seq][n_tokens][128] with the prefill outlier model; keys rotated."""
    g = _gen(seed, device)
    pos = torch.arange(n_tokens, device=device)[None, :].expand(n_seq, n_tokens)
    k = torch.empty((n_layers, n_heads, n_seq, n_tokens, HEAD_DIM), device=device, dtype=dtype)
    v = torch.empty_like(k)
    for layer in range(n_layers):
        for dst, rp in ((k, pos), (v, None)):
            x = outlier_heads(g, n_heads, n_seq, n_tokens, n_out_ch=3, ch_scale=20.0, rope_pos=rp, device=device)
            dst[layer] = x.to(dtype)
    return k, v


def decode_attn_layer(gen: torch.Generator, n_seq: int = 16, n_kv_heads: int = 8, n_q_heads: int = 32,
                      n_tokens: int = 32768, n_planted: int = 8, target_logit: float = 10.0, device="cuda",
                      dtype=torch.bfloat16):
    """One layer of the decode-attention workload.

    Returns (q fp16 [n_seq][n_q_heads][128], K, V [n_seq][n_kv_heads][n_tokens][128]).
    K and V follow the prefill outlier model (keys rotated at positions
    0..n_tokens-1).  In every (sequence, KV head), n_planted random tokens get the
    key alpha * mean of the group's queries, with alpha chosen so that the
    group's mean logit on them is target_logit: the softmax is peaked, as it is
    when a decode step attends to a few relevant tokens.
    """
    gs = n_q_heads // n_kv_heads
    q = torch.randn((n_seq, n_q_heads, HEAD_DIM), generator=gen, device=device).to(torch.float16)
    pos = torch.arange(n_tokens, device=device)[None, :].expand(n_seq, n_tokens)
    k = outlier_heads(gen, n_kv_heads, n_seq, n_tokens, n_out_ch=3, ch_scale=20.0, rope_pos=pos,
                      device=device).transpose(0, 1)
    v = outlier_heads(gen, n_kv_heads, n_seq, n_tokens, n_out_ch=3, ch_scale=20.0, device=device).transpose(0, 1)
    qm = q.float().view(n_seq, n_kv_heads, gs, HEAD_DIM).mean(dim=2)          # [seq][kv][128]
    alpha = target_logit * math.sqrt(HEAD_DIM) / (qm * qm).sum(-1).clamp_min(1e-6)  # [seq][kv]
    where = torch.argsort(torch.rand((n_seq, n_kv_heads, n_tokens), generator=gen, device=device),
                          dim=-1)[..., :n_planted]
    planted = (alpha[..., None] * qm)[:, :, None, :].expand(n_seq, n_kv_heads, n_planted, HEAD_DIM)
    k.scatter_(2, where[..., None].expand(-1, -1, -1, HEAD_DIM), planted.contiguous())
    return q, k.to(dtype).contiguous(), v.to(dtype).contiguous()


def generator(seed: int, device) -> torch.Generator:
    return _gen(seed, device)
