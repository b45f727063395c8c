"""Throughput of the KVarN codec on one MI355X.

Headline step = quantise + dequantise the whole KV cache of the Phi-4-14B
preset: 40 layers x 10 KV heads x 8 sequences x 16384 tokens, head_dim 128,
bf16 K and V (dense [layer][head][seq][token][128]), 4-bit keys and 2-bit
values (the released kvarn_k4v2_g128 preset) -- 409600 K tiles and 409600 V
tiles.  Inputs are resident in HBM before timing.

value = fp16-equivalent bytes moved by the step (819200 tiles x 32 KiB read by
the quantiser + the same written by the dequantiser) / step time.  The
roofline object describes the dominant kernel, the quantiser: algorithmic HBM
bytes per launch (tiles x (32768 + record bytes)) over its mean launch time
from HIP events around every launch (at least 20 per op), against 8 TB/s; the
same launches' algorithmic fp32 rate against the fp32 vector peak is reported
beside it.

Also in the line, each timed in the same run: the codec on the decode-append
block and on the bulk-prefill cache of the Qwen3-4B shape (secondary
workloads), decode attention over the packed cache at the Qwen3-4B shape (2-bit
K and V) and at the Phi-4 shape (4-bit K, 2-bit V), the method variants
(n_iter = 4 sensitivity row, Hadamard-only, KIVI), the second scale's
dequantisation cost, error statistics of the variants, a plain 256 MiB copy (the
achievable-bandwidth reference), and the oracle timed on the host on a bounded
sample of the headline workload plus a slice of one decode-attention layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_quantization_x128_amd import kvarn, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
# Published fp32 vector peak.  The library is built without packed fp32, but a
# plain (non-packed) wave64 v_fmac_f32 issues every 2.4-2.7 cycles on gfx950 when
# its two source VGPRs sit in different banks (measured with a probe kernel at
# 4-8 waves per SIMD): 256 CUs x 4 SIMDs x 64 lanes x 2 flops / 2 cycles x
# 2.4 GHz = 157.3 TFLOP/s is reachable without packed math.
FP32_VECTOR_PEAK_TFLOPS = 157.3
TILE_F16_BYTES = 128 * 128 * 2


def quantize_flops_per_tile(axis, n_iter=8):
    """Algorithmic fp32 operations of quantising one 128 x 128 tile.

    per element: rotation 7 butterfly add/sub + 1 scale = 8; each normalisation
    half-step 1 multiply by the factor + 1 add (sum) + 1 FMA (sum of squares, 2) = 4,
    2 * n_iter half-steps for K, 2 * n_iter - 1 for V (the last token factor of V
    is absorbed into s1 and never needed); metadata and codes: Zn multiply 1, group
    min and max 2, (Zn - z) / s1 as one FMA 2 = 5.
    """
    half_steps = 2 * n_iter - (1 if axis == kvarn.AXIS_V and n_iter > 0 else 0)
    return 128 * 128 * (8 + 4 * half_steps + 5)


CSRC = os.path.join(ROOT, "kv_cache_quantization_x128_amd", "csrc")
TRAFFIC = {"phi4": os.path.join(ROOT, "profiles", "traffic_phi4_k4v2.json"),
           "decode_append": os.path.join(ROOT, "profiles", "traffic_decode_append.json")}
KERNEL_SOURCES = {"quantize": ("quantize.hip", "kvarn_device.h"), "quantize_k": ("quantize.hip", "kvarn_device.h"),
                  "quantize_v": ("quantize.hip", "kvarn_device.h"),
                  "dequantize": ("dequantize.hip", "kvarn_device.h"), "dequantize_k": ("dequantize.hip", "kvarn_device.h"),
                  "dequantize_v": ("dequantize.hip", "kvarn_device.h"),
                  "decode_mfma": ("decode_attn.hip", "kvarn_device.h")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel, workload="decode_append"):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
    (scaled by the copy-kernel calibration), or None when the kernel's sources have
    changed since the counters were taken."""
    import hashlib
    import json as _json

    try:
        rec = _json.load(open(TRAFFIC[workload]))
        k = rec["kernels"][kernel]
        cal = rec["calibration"]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    if h.hexdigest()[:16] != k["source_sha256_16"]:
        return None
    return 1024 * (k["fetch_kib"] * cal["fetch_scale"] + k["write_kib"] * cal["write_scale"])


class OpTimer:
    """Accumulates HIP-event time of launches on the current stream."""

    def __init__(self):
        self.pairs = []

    def __call__(self, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def times_ms(self):
        torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs]

    def mean_ms(self):
        t = self.times_ms()
        return float(np.mean(t)) if t else float("nan")

    def stats(self):
        t = self.times_ms()
        return {"launches": len(t), "mean_ms": float(np.mean(t)), "median_ms": float(np.median(t)),
                "min_ms": float(np.min(t)), "max_ms": float(np.max(t))}


EVENT_EVERY = 10   # decode-append codec steps per step timed launch by launch
MIN_EVENTED = 20   # evented launches per op of the headline workload, whatever --steps is
DECODE_WARMUP_S = 0.5   # seconds of graph replays before decode attention is timed
CPU_SAMPLE = 4096  # headline tiles per cache the host oracle is timed on (8192 in all)

PHI4 = dict(layers=40, heads=10, seqs=8, tokens=16384, bits_k=4, bits_v=2)


def bench_phi4(steps, warmup):
    """The headline step on the Phi-4-14B preset caches (see the module docstring).
    HIP events bracket every launch of the timed steps (a launch takes
    milliseconds, an event microseconds); when --steps is below MIN_EVENTED,
    further evented steps follow the timed region so that every op has at least
    MIN_EVENTED launch timings."""
    dev = torch.device("cuda:0")
    c = PHI4
    log(f"generating the Phi-4 preset caches {c['layers']}x{c['heads']}x{c['seqs']}x{c['tokens']}x128 bf16")
    k, v = synth.phi4(n_layers=c["layers"], n_heads=c["heads"], n_seq=c["seqs"], n_tokens=c["tokens"], device=dev)
    n = k.numel() // (128 * 128)
    bk, bv = c["bits_k"], c["bits_v"]
    rk = torch.empty((n, kvarn.tile_bytes(bk)), dtype=torch.uint8, device=dev)
    rv = torch.empty((n, kvarn.tile_bytes(bv)), dtype=torch.uint8, device=dev)
    ok = torch.empty_like(k)
    ov = torch.empty_like(v)
    ops = (("quantize_k", lambda: kvarn.quantize_tiles(k, n, bk, kvarn.AXIS_K, out=rk)),
           ("quantize_v", lambda: kvarn.quantize_tiles(v, n, bv, kvarn.AXIS_V, out=rv)),
           ("dequantize_k", lambda: kvarn.dequantize_tiles(rk, n, bk, kvarn.AXIS_K, ok)),
           ("dequantize_v", lambda: kvarn.dequantize_tiles(rv, n, bv, kvarn.AXIS_V, ov)))
    timers = {name: OpTimer() for name, _ in ops}

    def step(timed):
        for name, fn in ops:
            timers[name](fn) if timed else fn()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {steps} headline steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for _ in range(max(0, MIN_EVENTED - steps)):
        step(True)
    per_op = {name: t.stats() for name, t in timers.items()}
    # the seeded tile sample the host oracle is timed on: exact bf16 bytes of
    # CPU_SAMPLE tiles of each cache, spread over layer, head and sequence
    rng = np.random.default_rng(4)
    sample = {}
    for name, x in (("k", k), ("v", v)):
        idx = torch.from_numpy(np.sort(rng.choice(n, size=CPU_SAMPLE, replace=False))).to(dev)
        sample[name] = x.view(n, 128, 128)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    alg = {"quantize_k": n * (TILE_F16_BYTES + kvarn.tile_bytes(bk)), "quantize_v": n * (TILE_F16_BYTES + kvarn.tile_bytes(bv))}
    alg["dequantize_k"], alg["dequantize_v"] = alg["quantize_k"], alg["quantize_v"]
    for name, st in per_op.items():
        st["algorithmic_bytes_per_launch"] = alg[name]
        st["algorithmic_GBs"] = alg[name] / (st["mean_ms"] * 1e-3) / 1e9
        st["frac_hbm"] = st["algorithmic_GBs"] / HBM_PEAK_GBS
        st["tiles_per_s"] = n / (st["mean_ms"] * 1e-3)
        st["bits"] = bk if name.endswith("_k") else bv
    del k, v, rk, rv, ok, ov
    torch.cuda.empty_cache()
    return dict(n_tiles_per_cache=n, wall_s=wall, per_op=per_op, sample=sample)


def bench_codec(steps, warmup, layers=36, seqs=64, heads=8, bits=2, with_variants=True):
    dev = torch.device("cuda:0")
    log(f"generating decode-append inputs {layers}x{seqs}x128x{heads}x128 bf16")
    k, v = synth.decode_append(n_layers=layers, n_seq=seqs, n_heads=heads, device=dev)
    offs = synth.decode_append_offsets(layers, seqs, heads, device=dev)
    n = offs.numel()
    ts = heads * 128
    pb = kvarn.tile_bytes(bits)
    rk = torch.empty((n, pb), dtype=torch.uint8, device=dev)
    rv = torch.empty_like(rk)
    ok = torch.empty_like(k)
    ov = torch.empty_like(v)
    timers = {name: OpTimer() for name in ("quantize_k", "quantize_v", "dequantize_k", "dequantize_v")}

    def step(timed):
        ops = (
            ("quantize_k", lambda: kvarn.quantize_tiles(k, n, bits, kvarn.AXIS_K, token_stride=ts, tile_offset=offs,
                                                        out=rk)),
            ("quantize_v", lambda: kvarn.quantize_tiles(v, n, bits, kvarn.AXIS_V, token_stride=ts, tile_offset=offs,
                                                        out=rv)),
            ("dequantize_k", lambda: kvarn.dequantize_tiles(rk, n, bits, kvarn.AXIS_K, ok, token_stride=ts,
                                                            dst_offset=offs)),
            ("dequantize_v", lambda: kvarn.dequantize_tiles(rv, n, bits, kvarn.AXIS_V, ov, token_stride=ts,
                                                            dst_offset=offs)),
        )
        for name, fn in ops:
            if timed:
                timers[name](fn)
            else:
                fn()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {steps} steps")
    # Every tenth step carries HIP events around each launch: each recorded
    # event costs the stream a few microseconds, so events on every launch
    # would add ~4 % to the step they are meant to describe.
    t0 = time.perf_counter()
    for i in range(steps):
        step(i % EVENT_EVERY == 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {name: t.mean_ms() for name, t in timers.items()}

    # Dequantisation with its records evicted from the memory-side cache first:
    # inside a step the records were written just before and can still be in
    # the 256 MB Infinity Cache.  A 1 GiB read-only pass (untimed) precedes
    # every timed launch here.
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    cold = OpTimer()
    for i in range(max(4, steps // 10)):
        for rec, out, axis in ((rk, ok, kvarn.AXIS_K), (rv, ov, kvarn.AXIS_V)):
            torch.sum(junk, dim=0, out=acc)
            cold(lambda: kvarn.dequantize_tiles(rec, n, bits, axis, out, token_stride=ts, dst_offset=offs))  # noqa
    per_op["dequantize_cold"] = cold.mean_ms()
    del junk

    # Method variants on the same K tiles: the method, Hadamard-only (no
    # normalisation) and KIVI (no rotation, no normalisation).
    variants = {}
    for name, n_iter, flags in (("kvarn", 8, 0), ("kvarn_n_iter_4", 4, 0), ("hadamard_only", 0, 0),
                                ("kivi", 0, kvarn.NO_ROTATION)):
        if not with_variants:
            break
        tq, td = OpTimer(), OpTimer()
        for i in range(max(4, steps // 10) + 2):
            fq = lambda: kvarn.quantize_tiles(k, n, bits, kvarn.AXIS_K, token_stride=ts, tile_offset=offs,  # noqa
                                              out=rk, n_iter=n_iter, flags=flags)
            fd = lambda: kvarn.dequantize_tiles(rk, n, bits, kvarn.AXIS_K, ok, token_stride=ts,  # noqa
                                                dst_offset=offs, flags=flags)
            tq(fq) if i >= 2 else fq()
            td(fd) if i >= 2 else fd()
        variants[name] = {"n_iter": n_iter, "rotation": not flags, "quantize_k_ms": tq.mean_ms(),
                          "dequantize_k_ms": td.mean_ms()}
    return dict(n_tiles_per_cache=n, bits=bits, wall_s=wall, per_op_ms=per_op, record_bytes=pb, variants=variants)


def bench_other_workloads(reps=5):
    """Per-launch rates of the codec on the bulk-prefill cache of the Qwen3-4B
    shape (36 layers x 8 KV heads x 32768 tokens, dense, 2-bit K and V).  Whole
    caches, one launch per cache and op, HIP events around each of `reps`
    launches after one untimed launch."""
    dev = torch.device("cuda:0")
    res = {}
    for name, gen, bits_k, bits_v in (("prefill_qwen3_4b", synth.prefill, 2, 2),):
        log(f"generating {name} inputs")
        k, v = gen(device=dev)
        n = k.numel() // (128 * 128)
        out = torch.empty_like(k)
        ops = {}
        for cache, x, axis, bits in (("k", k, kvarn.AXIS_K, bits_k), ("v", v, kvarn.AXIS_V, bits_v)):
            rec = torch.empty((n, kvarn.tile_bytes(bits)), dtype=torch.uint8, device=dev)
            tq, td = OpTimer(), OpTimer()
            for i in range(reps + 1):
                fq = lambda: kvarn.quantize_tiles(x, n, bits, axis, out=rec)  # noqa: E731
                fd = lambda: kvarn.dequantize_tiles(rec, n, bits, axis, out)  # noqa: E731
                tq(fq) if i else fq()
                td(fd) if i else fd()
            alg = n * (32768 + kvarn.tile_bytes(bits))
            for op, t in (("quantize_" + cache, tq.mean_ms()), ("dequantize_" + cache, td.mean_ms())):
                ops[op] = {"bits": bits, "launch_ms": t, "tiles_per_s": n / (t * 1e-3),
                           "fp16_equiv_GBs": n * 32768 / (t * 1e-3) / 1e9,
                           "algorithmic_GBs": alg / (t * 1e-3) / 1e9,
                           "frac_hbm": alg / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del rec
        total_ms = sum(o["launch_ms"] for o in ops.values())
        res[name] = {"tiles_per_cache": n, "ops": ops,
                     "quantize_plus_dequantize_fp16_equiv_GBs": 4 * n * 32768 / (total_ms * 1e-3) / 1e9}
        del k, v, out
        torch.cuda.empty_cache()
    return res


TOPK_PCTS = (0.1, 1.0, 5.0, 10.0, 25.0, 50.0)
HIST_EDGES = tuple(float(e) for e in np.arange(0.0, 9.01, 0.5))    # log2 of token norms, 18 bins


def error_analysis(x: torch.Tensor, xd: torch.Tensor) -> dict:
    """Error statistics of dequantised key vectors xd against the originals x
    (rows = tokens, 128 channels), in float64.

    * Per token, the error splits exactly into a magnitude and a direction part
      (pheeree.github.io blog, part 2, equation 3; paperlayer.ai summary,
      section 3 Methods, error decomposition):
          |x - xd|^2 = (|x| - |xd|)^2 + 2 |x| |xd| (1 - cos theta) = E_M + E_D;
      reported as the magnitude share E_M / E_T summed over the tokens with the
      largest q of the errors (q = 50 % ... 0.1 %).
    * Outlier contributions (appendix C): the entries ranked by squared error;
      the share of the squared error left after replacing the largest k % of
      the entries with exact values ("top_fixed") and after replacing the other
      (100 - k) % ("bottom_fixed"), for k in TOPK_PCTS.
    * Token scales (appendix B): the joint distribution of (log2 |x|,
      log2 |xd|) over the tokens as a 2-D histogram on HIST_EDGES (rows: before,
      columns: after quantisation), the fraction of tokens off the diagonal by
      more than 0.1 / 0.25 / 0.5 / 1 in log2, and the mean |log2(|xd| / |x|)|
      overall and for the 5 % of tokens with the largest and the smallest norms."""
    x, xd = x.double(), xd.double()
    nk, nd = x.norm(dim=1), xd.norm(dim=1)
    e_t = ((x - xd) ** 2).sum(1)
    e_m = (nk - nd) ** 2
    order = torch.argsort(e_t, descending=True)
    shares = {}
    for q in (0.5, 0.1, 0.05, 0.01, 0.001):
        top = order[:max(1, int(round(q * e_t.numel())))]
        shares[f"top_{q * 100:g}pct"] = float(e_m[top].sum() / e_t[top].sum())
    el = ((x - xd) ** 2).reshape(-1)
    el_sorted = torch.sort(el, descending=True).values
    total = float(el_sorted.sum())
    total = total if total > 0 else 1.0             # exact reconstruction: every share is 0
    csum = torch.cumsum(el_sorted, 0)
    residual = {}
    for k in TOPK_PCTS:
        m = max(1, int(round(k / 100 * el.numel())))
        top_sum = float(csum[m - 1])
        residual[f"{k:g}pct"] = {"top_fixed": (total - top_sum) / total, "bottom_fixed": top_sum / total}
    lk = torch.log2(nk.clamp_min(1e-300))
    ld = torch.log2(nd.clamp_min(1e-300))
    scale = (ld - lk).abs()
    edges = torch.tensor(HIST_EDGES, dtype=torch.float64, device=x.device)
    nb = len(HIST_EDGES) - 1
    bi = (torch.bucketize(lk, edges, right=True) - 1).clamp(0, nb - 1)
    bj = (torch.bucketize(ld, edges, right=True) - 1).clamp(0, nb - 1)
    hist = torch.zeros(nb * nb, dtype=torch.int64, device=x.device)
    hist.index_add_(0, bi * nb + bj, torch.ones_like(bi))
    by_norm = torch.argsort(nk)
    k5 = max(1, int(round(0.05 * nk.numel())))
    return {"rel_mse": float(e_t.sum() / (x * x).sum()),
            "magnitude_share": {k: (v if v == v else 0.0) for k, v in shares.items()},
            "top5pct_entries_share_of_sq_error": residual["5pct"]["bottom_fixed"],
            "residual_sq_error_share": residual,
            "token_scale_abs_log2": {"mean": float(scale.mean()), "largest_5pct_norms": float(scale[by_norm[-k5:]].mean()),
                                     "smallest_5pct_norms": float(scale[by_norm[:k5]].mean())},
            "token_scale_off_diagonal": {f"gt_{t:g}": float((scale > t).double().mean()) for t in (0.1, 0.25, 0.5, 1.0)},
            "token_scale_joint_hist": {"log2_edges": list(HIST_EDGES), "counts": hist.view(nb, nb).cpu().tolist(),
                                       "rows": "log2 |x| before", "columns": "log2 |xd| after"}}


def bench_error_analysis(n_layers=4, bits=2):
    """KVarN vs Hadamard-only vs KIVI on the keys of the decode-append workload
    (first n_layers layers: 64 sequences x 8 KV heads, one 128-token tile each)."""
    dev = torch.device("cuda:0")
    k, _ = synth.decode_append(n_layers=n_layers, n_seq=64, n_heads=8, device=dev)
    tiles = k.permute(0, 1, 3, 2, 4).contiguous()                        # [L][seq][head][128 tok][128 ch]
    n = tiles.numel() // (128 * 128)
    x = tiles.view(n * 128, 128).float()
    out = {"workload": f"keys of the decode-append workload, {n} tiles ({n_layers} layers), {bits}-bit"}
    for name, n_iter, flags in (("kvarn", 8, 0), ("hadamard_only", 0, 0), ("kivi", 0, kvarn.NO_ROTATION)):
        rec = kvarn.quantize(tiles, bits, kvarn.AXIS_K, n_iter=n_iter, flags=flags)
        xd = kvarn.dequantize(rec, bits, kvarn.AXIS_K, torch.float32, flags=flags).view(n * 128, 128)
        out[name] = error_analysis(x, xd)
    return out


def _interleaved_graph_us(calls: dict, reps=20, rounds=9) -> dict:
    """Median time per call of each entry of `calls`: each is captured in a HIP
    graph of `reps` calls; after a shared warm-up the graphs are timed in turn,
    round after round, so that clock drift falls on all of them alike."""
    graphs = {}
    for name, call in calls.items():
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                call()
        graphs[name] = g
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < DECODE_WARMUP_S:
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
    times = {name: [] for name in graphs}
    for _ in range(rounds):
        for name, g in graphs.items():
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            g.replay()
            e0.record()
            torch.cuda.synchronize()
            times[name].append(s0.elapsed_time(e0) * 1e3 / reps)
    del graphs
    return {name: float(np.median(t)) for name, t in times.items()}


def bench_app_i(contexts=(4096, 8192, 16384, 32768), heads=16):
    """The second scale's cost at the shape of the pages' dequantisation-overhead
    measurement (paperlayer.ai summary, appendix I: 16 attention heads, head_dim
    128, groups of 128, 4k-32k tokens, one query token).  KIVI records (no
    rotation, no normalisation, s2 = 1/2) go through the same kernels twice:
    with the dual-scale path (the s2 block read and applied, as for KVarN
    records) and with KVARN_SINGLE_SCALE (no s2 read, one FMA per element), so
    the difference is the second scale alone; KVarN records (with the rotation)
    are timed beside them.  Both the fused decode-attention read and the
    standalone dequantisation of the K and V records are timed, as the median
    time per call over HIP-graph replays, the six graphs of a context timed in
    turn after a shared warm-up."""
    dev = torch.device("cuda:0")
    g = synth.generator(1006, dev)
    nr, ss = kvarn.NO_ROTATION, kvarn.NO_ROTATION | kvarn.SINGLE_SCALE
    rows = []
    for T in contexts:
        nt = T // 128
        q, kx, vx = synth.decode_attn_layer(g, n_seq=1, n_kv_heads=heads, n_q_heads=heads, n_tokens=T, device=dev)
        n_tiles = torch.full((1,), nt, dtype=torch.int32, device=dev)
        recs = {"kvarn": (kvarn.quantize(kx, 2, kvarn.AXIS_K), kvarn.quantize(vx, 2, kvarn.AXIS_V)),
                "kivi": (kvarn.quantize(kx, 2, kvarn.AXIS_K, n_iter=0, flags=nr),
                         kvarn.quantize(vx, 2, kvarn.AXIS_V, n_iter=0, flags=nr))}
        ws = torch.empty(kvarn.workspace_bytes(1, heads, heads, nt), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        ok, ov = torch.empty_like(kx), torch.empty_like(vx)
        row = {"tokens": T}
        calls = {}
        for name, rname, flags in (("kvarn", "kvarn", 0), ("kivi_dual_scale", "kivi", nr),
                                   ("kivi_single_scale", "kivi", ss)):
            kr, vr = recs[rname]
            n = kr.shape[0]
            calls[f"decode_{name}_us"] = (
                lambda kr=kr, vr=vr, flags=flags: kvarn.decode_attn(q, kr, vr, n_tiles, heads, nt, 2, 2, out=out,
                                                                    workspace=ws, flags=flags))
            calls[f"dequant_{name}_us"] = (
                lambda kr=kr, vr=vr, n=n, flags=flags: (kvarn.dequantize_tiles(kr, n, 2, kvarn.AXIS_K, ok, flags=flags),
                                                        kvarn.dequantize_tiles(vr, n, 2, kvarn.AXIS_V, ov, flags=flags)))
        row.update(_interleaved_graph_us(calls))
        for what in ("decode", "dequant"):
            single = row[f"{what}_kivi_single_scale_us"]
            row[f"{what}_second_scale_pct"] = 100.0 * (row[f"{what}_kivi_dual_scale_us"] / single - 1.0)
            row[f"{what}_kvarn_over_kivi_single_pct"] = 100.0 * (row[f"{what}_kvarn_us"] / single - 1.0)
        rows.append(row)
    return {"what": "the second scale's cost: KIVI records through the dual-scale path (s2 read and applied) and "
                    "the single-scale path (KVARN_SINGLE_SCALE), and KVarN records, 16 heads, head_dim 128, one "
                    "query token; fused decode-attention read and standalone K + V dequantisation; median time "
                    "per call over HIP-graph replays",
            "pages": "at most 1.4 % between KVarN and KIVI dequantisation at 4k-32k tokens, within noise at 16k "
                     "and 32k (paperlayer.ai summary, appendix I; Triton kernels on other hardware)",
            "rows": rows}


def warm_replays(graph, n_min):
    """Replay `graph` at least n_min times and for at least DECODE_WARMUP_S
    seconds: the timed replays last tens of milliseconds, and after host-paced
    work the GPU needs a few hundred milliseconds of load to reach its
    sustained clock (decode attention, latency-bound, ran 5-7 % slower without)."""
    t0 = time.perf_counter()
    n = 0
    while n < n_min or time.perf_counter() - t0 < DECODE_WARMUP_S:
        graph.replay()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def bench_decode(passes, warmup, layers=36, batch=16, hq=32, hkv=8, tokens=32768, bits=2, bits_v=None,
                 with_windows=True, seed=1005):
    """Decode attention over packed caches of `layers` distinct layers (one
    query token per sequence), 2-bit K and V by default, `bits_v` for other V
    widths."""
    dev = torch.device("cuda:0")
    nt = tokens // 128
    bk, bv = bits, (bits if bits_v is None else bits_v)
    g = synth.generator(seed, dev)
    caches = []
    log(f"building {layers} decode-attention layers (batch {batch}, {hq}/{hkv} heads, {tokens} tokens, K{bk}V{bv})")
    for _ in range(layers):
        q, k, v = synth.decode_attn_layer(g, n_seq=batch, n_kv_heads=hkv, n_q_heads=hq, n_tokens=tokens, device=dev)
        caches.append((q, kvarn.quantize(k, bk, kvarn.AXIS_K), kvarn.quantize(v, bv, kvarn.AXIS_V)))
        del k, v
    torch.cuda.empty_cache()
    n_tiles = torch.full((batch,), nt, dtype=torch.int32, device=dev)
    ws = torch.empty(kvarn.workspace_bytes(batch, hq, hkv, nt), dtype=torch.uint8, device=dev)
    out = torch.empty((batch, hq, 128), dtype=torch.float16, device=dev)
    timer = OpTimer()

    def one_pass(timed):
        for q, kr, vr in caches:
            fn = lambda: kvarn.decode_attn(q, kr, vr, n_tiles, hkv, nt, bk, bv, out=out, workspace=ws)  # noqa
            timer(fn) if timed else fn()

    # eager: HIP events around every call (includes the host's launch overhead
    # whenever the host is slower than the GPU)
    for _ in range(warmup):
        one_pass(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(passes):
        one_pass(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = timer.mean_ms()
    ref = out.clone()
    # the same pass captured once in a HIP graph and replayed: device time per layer
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass(False)
    # timed straight after the warm-up: an idle gap of a few tens of milliseconds
    # (a host-side check here took ~37 ms) drops the clock, and the first
    # replays after it ran at 67 instead of 48 us per decode kernel
    warm_replays(graph, warmup)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(passes):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    layer_ms = s.elapsed_time(e) / (passes * layers)
    if not torch.equal(out, ref):
        raise RuntimeError("decode attention: graph replay differs from the eager pass")
    del graph

    alg_bytes = batch * hkv * nt * (kvarn.tile_bytes(bk) + kvarn.tile_bytes(bv)) + 2 * batch * hq * 128 * 2
    ach = alg_bytes / (layer_ms * 1e-3) / 1e9
    res = {
        "workload": f"decode attention: batch {batch}, {hq} query heads on {hkv} KV heads, head_dim 128, "
                    f"{tokens}-token cache, {bk}-bit K, {bv}-bit V, {layers} layers",
        "layer_ms": layer_ms,
        "timing": f"HIP events around {passes} replays of a HIP graph holding the {layers}-layer pass",
        "eager_layer_ms": eager_ms,
        "eager_wall_s_per_pass": wall / passes,
        "fp16_equiv_GBs": 2 * batch * hkv * nt * TILE_F16_BYTES / (layer_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS,
                     "traffic": ({(2, 2, 16, 32, 8, 32768): lambda: measured_traffic("decode_mfma"),
                                  (4, 2, 8, 40, 10, 16384): lambda: measured_traffic("decode_mfma", "phi4")}
                                 .get((bk, bv, batch, hq, hkv, tokens), lambda: None)()),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "tokens_per_s": batch * hq / (layer_ms * 1e-3),
    }
    if not with_windows:
        return res

    # The same layers with the pages' FP16 windows around the packed body: 128
    # sink tokens and a trailing window of capacity 128 holding 1-128 tokens.
    n_sink, cap = 128, 128
    wins = []
    for _ in range(layers):
        w = [torch.randn((batch, hkv, n, 128), generator=g, device=dev).to(torch.float16)
             for n in (n_sink, n_sink, cap, cap)]
        wins.append(w)
    n_recent = torch.randint(1, cap + 1, (batch,), generator=g, device=dev, dtype=torch.int32)

    def window_pass():
        for (q, kr, vr), (ks, vs, kt, vt) in zip(caches, wins):
            kvarn.decode_attn(q, kr, vr, n_tiles, hkv, nt, bk, bv, out=out, workspace=ws, k_sink=ks, v_sink=vs,
                              k_recent=kt, v_recent=vt, n_recent=n_recent)

    window_pass()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        window_pass()
    warm_replays(graph, warmup)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(passes):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    win_ms = s.elapsed_time(e) / (passes * layers)
    del graph, wins
    win_tokens = batch * (n_sink + float(n_recent.float().mean()))
    res["with_fp16_windows"] = {
        "layer_ms": win_ms, "sink_tokens": n_sink, "recent_capacity": cap,
        "mean_recent_tokens": win_tokens / batch - n_sink,
        "extra_bytes_per_layer": 2 * hkv * win_tokens * 256,
        "note": "same layers, attention also over FP16 sink (128) and trailing (1-128) tokens per sequence",
    }
    return res


def copy_reference(reps=10, nbytes=1 << 28):
    """A plain elementwise copy (one dispatch, fp32, read nbytes + write nbytes): the
    achievable-bandwidth reference, and the calibration of the profiler's
    FETCH/WRITE counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    t = OpTimer()
    for _ in range(reps):
        t(lambda: torch.mul(src, 1.0, out=dst))
    ms = t.mean_ms()
    return {"kernel": "torch elementwise mul-by-1 copy", "bytes_per_launch": 2 * nbytes, "launch_ms": ms,
            "GBs": 2 * nbytes / (ms * 1e-3) / 1e9}


def host_info():
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_in_affinity_mask": len(os.sched_getaffinity(0))}


def cpu_baseline(sample, n_full, min_s=10.0, max_passes=12):
    """The oracle's quantise + dequantise of the headline workload's seeded tile
    sample (CPU_SAMPLE K tiles at 4 bits + CPU_SAMPLE V tiles at 2 bits, the
    exact bf16 bytes of the GPU's inputs), repeated until at least min_s of host
    work, in the headline's unit (fp16-equivalent GB/s of quantise + dequantise);
    the whole step's host time is extrapolated from it."""
    import oracle

    def one_pass():
        t0 = time.perf_counter()
        for key, axis, bits in (("k", oracle.AXIS_K, PHI4["bits_k"]), ("v", oracle.AXIS_V, PHI4["bits_v"])):
            rec = oracle.quantize(oracle.TileView.dense(sample[key], oracle.DT_BF16), bits, axis)
            oracle.dequantize(rec, bits, axis)
        return time.perf_counter() - t0

    dt, passes = one_pass(), 1
    while dt < min_s and passes < max_passes:
        dt += one_pass()
        passes += 1
    m = sample["k"].shape[0]
    per_pass = dt / passes
    return {"value": passes * 2 * (2 * m) * TILE_F16_BYTES / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", **host_info(),
            "sample": f"{m} K tiles (4-bit) + {m} V tiles (2-bit) of the Phi-4 preset caches (seeded, over layer, head "
                      f"and sequence), quantise + dequantise, {passes} passes, {dt:.1f} s on the host",
            "extrapolated_step_s": per_pass * n_full / m,
            "extrapolation": f"the whole headline step ({n_full} K + {n_full} V tiles) at the sample's rate"}


def cpu_decode_layer(n_seq_sample=16, batch=16, hq=32, hkv=8, tokens=32768):
    """The oracle's decode attention on one layer of the Qwen3-4B decode
    workload (by default all of the batch's sequences, KV heads and tiles;
    records written by the oracle itself, untimed); a slice of n_seq_sample
    sequences is extrapolated to the whole layer."""
    import oracle

    g = synth.generator(1005, "cpu")
    q, k, v = synth.decode_attn_layer(g, n_seq=n_seq_sample, n_kv_heads=hkv, n_q_heads=hq, n_tokens=tokens,
                                      device="cpu")
    bits16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1, 128, 128)  # noqa: E731
    kr = oracle.quantize(oracle.TileView.dense(bits16(k), oracle.DT_BF16), 2, oracle.AXIS_K)
    vr = oracle.quantize(oracle.TileView.dense(bits16(v), oracle.DT_BF16), 2, oracle.AXIS_V)
    nt = tokens // 128
    t0 = time.perf_counter()
    oracle.decode_attn(q.numpy().view(np.uint16), kr, vr, np.full(n_seq_sample, nt, np.int32), hq, hkv, nt, 2, 2)
    dt = time.perf_counter() - t0
    return {"layer_s": dt * batch / n_seq_sample, "unit": "s per layer", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": (f"the whole layer: {batch} sequences x {hkv} KV heads x {tokens} tokens (2-bit K and V), "
                       f"{dt:.1f} s on the host" if n_seq_sample == batch else
                       f"{n_seq_sample} of {batch} sequences x {hkv} KV heads x {tokens} tokens (2-bit K and V), "
                       f"{dt:.1f} s on the host, extrapolated to the layer's {batch} sequences")}


def pages_context(variants, q_ms, layers=36):
    """The pages' own cost figure for the normalisation, beside what it costs here
    on the decode-append block (paperlayer.ai summary, section 4 Experiments,
    Efficiency).  Other hardware and an unstated batch: context, not a target."""
    norm_ms = variants["kvarn"]["quantize_k_ms"] - variants["hadamard_only"]["quantize_k_ms"]
    return {
        "pages": "1.9 ms for the eight normalisation rounds against 1050 ms to generate 128 tokens (0.18 %), "
                 "Qwen3-4B served by vLLM in fp16 on a GPU of 500 TFLOP/s fp16 and 1.8 TB/s",
        "here_normalisation_ms": norm_ms,
        "here_normalisation_per_layer_us": norm_ms / layers * 1e3,
        "here_quantise_k_and_v_ms": 2 * q_ms,
        "here_what": "one 128-token block of 64 sequences x 8 KV heads x 36 layers; normalisation = K quantise at "
                     "n_iter 8 minus n_iter 0 on the same tiles; quantise = the K and V launches of the step",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-passes", type=int, default=20)
    ap.add_argument("--decode-layers", type=int, default=36)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the decode-append and prefill codec workloads")
    ap.add_argument("--copy-calib", action="store_true",
                    help="time the plain 256 MiB device copy 10 times instead of 5 (counter calibration runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the method variants, the FP16-window decode, the KIVI comparison and the error "
                         "analysis (counter runs: every dispatch of a kernel is then a listed workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the codec has no cross-GPU step); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    kvarn.load()
    torch.cuda.init()

    # the small decode-append workload runs first, before the headline's 59 GB
    # of buffers have come and gone (its cold-dequantise timing, after a 1 GiB
    # read, is sensitive to how its buffers are mapped)
    codec = None if args.no_secondary else bench_codec(args.steps * 10, args.warmup * 3,
                                                       with_variants=not args.no_extras)
    head = bench_phi4(args.steps, args.warmup)
    n = head["n_tiles_per_cache"]
    per_op = head["per_op"]
    step_ms = head["wall_s"] / args.steps * 1e3
    f16_bytes = 2 * (2 * n) * TILE_F16_BYTES          # quantiser reads + dequantiser writes, K and V
    value = f16_bytes / (step_ms * 1e-3) / 1e9
    qk = per_op["quantize_k"]
    q_flops = n * quantize_flops_per_tile(kvarn.AXIS_K)
    q_tflops = q_flops / (qk["mean_ms"] * 1e-3) / 1e12
    ops = dict(per_op)
    t_q = per_op["quantize_k"]["mean_ms"] + per_op["quantize_v"]["mean_ms"]
    t_dq = per_op["dequantize_k"]["mean_ms"] + per_op["dequantize_v"]["mean_ms"]
    b_q = per_op["quantize_k"]["algorithmic_bytes_per_launch"] + per_op["quantize_v"]["algorithmic_bytes_per_launch"]
    ops["combined"] = {"what": "quantise + dequantise of the K and V caches: algorithmic bytes of all four launches over "
                               "the sum of their mean launch times",
                       "GBs": 2 * b_q / ((t_q + t_dq) * 1e-3) / 1e9,
                       "frac_hbm": 2 * b_q / ((t_q + t_dq) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "fp16_equiv_GBs": 4 * n * TILE_F16_BYTES / ((t_q + t_dq) * 1e-3) / 1e9}
    for name in ("quantize_k", "quantize_v", "dequantize_k", "dequantize_v"):
        ops[name]["traffic"] = measured_traffic(name, "phi4")
    line = {
        "metric": "KV quantize+dequant GB/s (fp16-equiv) and % of HBM peak on 1 MI355X",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1), 3 outlier channels x20 per (layer, head), 5% outlier tokens x4, "
                "RoPE-rotated keys; bf16)",
        "config": {"workload": "Phi-4-14B KV preset kvarn_k4v2_g128: 40 layers x 10 KV heads x 8 sequences x 16384 "
                               "tokens, head_dim 128, bf16 K and V, 4-bit K and 2-bit V",
                   "tiles_per_step": 2 * n, "layout": "[layer][head][seq][token][128]", "n_iter": 8,
                   "input_dtype": "bf16", "records": "4-bit K 8704 B, 2-bit V 4608 B per tile"},
        "frac_of_hbm_peak": value / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": "quantize_kernel<4, K, bf16, rotation> (the 409600 K tiles)",
                     "achieved": qk["algorithmic_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": qk["algorithmic_GBs"] / HBM_PEAK_GBS, "traffic": ops["quantize_k"]["traffic"],
                     "algorithmic_bytes_per_launch": qk["algorithmic_bytes_per_launch"],
                     "launch_ms_mean": qk["mean_ms"], "launch_ms_median": qk["median_ms"],
                     "launches_timed": qk["launches"],
                     "alu": {"what": "the same launches' algorithmic fp32 operations (quantize_flops_per_tile) against "
                                     "the fp32 vector peak, which non-packed FMAs reach when their sources sit in "
                                     "different register banks",
                             "achieved_TFLOPs": q_tflops, "peak_TFLOPs": FP32_VECTOR_PEAK_TFLOPS,
                             "frac": q_tflops / FP32_VECTOR_PEAK_TFLOPS,
                             "algorithmic_flops_per_launch": q_flops}},
        "ops": ops,
    }
    sample = head.pop("sample")
    if codec is not None:
        m = codec["n_tiles_per_cache"]
        pc = codec["per_op_ms"]
        sec_ms = codec["wall_s"] / (args.steps * 10) * 1e3
        q_ms = 0.5 * (pc["quantize_k"] + pc["quantize_v"])
        dq_ms = 0.5 * (pc["dequantize_k"] + pc["dequantize_v"])
        alg = m * (TILE_F16_BYTES + codec["record_bytes"])
        line["decode_append"] = {
            "workload": "Qwen3-4B KV shape, 36 layers x 64 sequences x 8 KV heads, one new 128-token block each, "
                        "bf16 token-major [layer][seq][token][head][128], 2-bit K and V",
            "tiles_per_step": 2 * m, "ms_per_step": sec_ms,
            "fp16_equiv_GBs": 2 * (2 * m) * TILE_F16_BYTES / (sec_ms * 1e-3) / 1e9,
            "quantize": {"launch_ms": q_ms, "algorithmic_GBs": alg / (q_ms * 1e-3) / 1e9,
                         "frac_hbm": alg / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "tiles_per_s": m / (q_ms * 1e-3),
                         "traffic": measured_traffic("quantize")},
            "dequantize": {"launch_ms": dq_ms, "algorithmic_GBs": alg / (dq_ms * 1e-3) / 1e9,
                           "frac_hbm": alg / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "traffic": measured_traffic("dequantize"),
                           "note": "inside the step: records written by the preceding quantise launches"},
            "dequantize_cold": {"launch_ms": pc["dequantize_cold"],
                                "frac_hbm": alg / (pc["dequantize_cold"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                "note": "records evicted from the memory-side cache before each launch"},
        }
        if not args.no_extras:
            line["variants_decode_append_k"] = codec["variants"]
            line["pages_context"] = pages_context(codec["variants"], q_ms)
            line["other_workloads"] = bench_other_workloads()
    if not args.no_decode:
        line["decode_attn"] = bench_decode(args.decode_passes, 2, layers=args.decode_layers,
                                           with_windows=not args.no_extras)
        line["decode_attn_phi4_k4v2"] = bench_decode(args.decode_passes, 2, layers=40, batch=8, hq=40, hkv=10,
                                                     tokens=16384, bits=4, bits_v=2, with_windows=False, seed=1007)
        if not args.no_extras:
            line["dequant_overhead_vs_kivi"] = bench_app_i()
            line["error_analysis"] = bench_error_analysis()
    line["copy_reference"] = copy_reference(reps=10 if args.copy_calib else 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(sample, n)
        line["cpu_baseline_decode_layer"] = cpu_decode_layer()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
