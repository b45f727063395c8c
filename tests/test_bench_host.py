"""Host-side pieces of bench.py that need no GPU: the algorithmic operation
count behind the quantiser's roofline, the traffic record's staleness check,
and the pages' context figure."""
import json
import os

import pytest

import bench
from kv_cache_quantization_x128_amd import kvarn


def test_quantize_flops_per_tile_against_the_survey_count():
    """The roofline's operation count against an independent count of one
    128 x 128 tile: the rotation's butterflies (7 stages of 16384 add/sub) plus
    the 1/sqrt(128) scale (16384 multiplies), 0.13 M; each normalisation
    half-step two matrix-vector products with the tile (the weighted sums of Y
    and of Y^2, one multiply-add = 2 flops per element each), 16 half-steps of
    2 x 16384 FMAs = 0.52 M FMAs for K; metadata and codes about 0.07 M.  The
    exact figure may differ from the estimate only in the ~0.07 M term."""
    rotation = 7 * 16384 + 16384
    half_step = 2 * 16384 * 2
    for axis, half_steps in ((kvarn.AXIS_K, 16), (kvarn.AXIS_V, 15)):
        est = rotation + half_steps * half_step + 70_000
        assert abs(bench.quantize_flops_per_tile(axis) - est) <= 0.02 * est
    # n_iter = 0 leaves the rotation and the codes only
    assert abs(bench.quantize_flops_per_tile(kvarn.AXIS_K, n_iter=0) - (rotation + 70_000)) <= 15_000
    # eight iterations cost twice the normalisation of four
    k8, k4, k0 = (bench.quantize_flops_per_tile(kvarn.AXIS_K, n_iter=t) for t in (8, 4, 0))
    assert k8 - k0 == 2 * (k4 - k0)


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    """A record whose source hashes match gives calibrated bytes; an edit of a
    hashed source, or no record, gives None (the bench then reports no traffic)."""
    import hashlib

    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for f in {f for fs in bench.KERNEL_SOURCES.values() for f in fs}:
        (csrc / f).write_bytes(open(os.path.join(bench.CSRC, f), "rb").read())

    def sha(kernel):
        h = hashlib.sha256()
        for f in bench.KERNEL_SOURCES[kernel]:
            h.update((csrc / f).read_bytes())
        return h.hexdigest()[:16]

    rec = {"calibration": {"fetch_scale": 2.0, "write_scale": 1.0},
           "kernels": {k: {"source_sha256_16": sha(k), "fetch_kib": 100.0 + i, "write_kib": 10.0}
                       for i, k in enumerate(bench.KERNEL_SOURCES)}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "TRAFFIC", {"decode_append": str(path)})
    for i, k in enumerate(bench.KERNEL_SOURCES):
        assert bench.measured_traffic(k) == pytest.approx(1024 * ((100.0 + i) * 2.0 + 10.0)), k
    (csrc / "quantize.hip").write_bytes((csrc / "quantize.hip").read_bytes() + b"\n")
    assert bench.measured_traffic("quantize") is None
    assert bench.measured_traffic("decode_mfma") is not None
    monkeypatch.setattr(bench, "TRAFFIC", {"decode_append": str(tmp_path / "missing.json")})
    assert bench.measured_traffic("decode_mfma") is None


def test_pages_context_is_the_normalisation_share():
    v = {"kvarn": {"quantize_k_ms": 0.5}, "hadamard_only": {"quantize_k_ms": 0.2}}
    ctx = bench.pages_context(v, 0.47)
    assert ctx["here_normalisation_ms"] == pytest.approx(0.3)
    assert ctx["here_normalisation_per_layer_us"] == pytest.approx(300.0 / 36)
    assert ctx["here_quantise_k_and_v_ms"] == pytest.approx(0.94)
    assert "1.9 ms" in ctx["pages"] and "0.18 %" in ctx["pages"]
