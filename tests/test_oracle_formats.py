"""Pins of the oracle's number formats against library routines and brute force.

FP8 E4M3 (OCP, "FN" variant) holds the two scales, FP16 the zero-point
(paperlayer.ai summary of arXiv 2606.03458v1, appendix D Experimental details:
two FP8 scales and one FP16 zero-point per 128-element group).
"""
import numpy as np
import pytest
import torch

pytestmark = []


def _fp8_table():
    """All finite non-negative FP8 E4M3 values, from torch's float8_e4m3fn (a library decoder)."""
    codes = torch.arange(128, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).double().numpy()
    keep = np.isfinite(vals)
    return codes.numpy()[keep], vals[keep]


def test_fp8_decode_all_codes_match_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.fp8_decode(int(c)) for c in range(256)])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.isnan(got).sum() == 2  # S.1111.111 only
    assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9


def test_fp8_encode_round_trips_every_code(orc):
    codes, vals = _fp8_table()
    for c, v in zip(codes, vals):
        assert orc.fp8_encode(v) == c
        assert orc.fp8_encode(-v) == (c | 0x80 if v != 0 else 0x80)


def test_fp8_encode_matches_brute_force_nearest(orc):
    """Nearest finite value, ties to the even code, saturating at 448."""
    codes, vals = _fp8_table()
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 4000)),
        (vals[1:] + vals[:-1]) / 2.0,  # every midpoint
        [0.0, 448.0, 449.0, 463.999, 464.0, 465.0, 1e6, 2.0 ** -10, 2.0 ** -11],
    ])
    for x in xs:
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:  # a tie: pick the even code
            pick = best[0] if codes[best[0]] % 2 == 0 else best[1]
        else:
            pick = best[0]
        assert orc.fp8_encode(x) == codes[pick], x


def test_fp8_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(8)
    xs = np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 20000)).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.fp8_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(ref, got)


def test_fp16_round_matches_numpy(orc):
    rng = np.random.default_rng(9)
    xs = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-20, 11, 20000)),
        rng.uniform(-65000, 65000, 2000),
    ])
    half = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (half[1:] + half[:-1]) / 2.0
    xs = np.concatenate([xs, mids[::7], -mids[::11]])
    xs = xs[np.abs(xs) < 65520.0]  # beyond, numpy overflows to inf while the oracle saturates
    ref = xs.astype(np.float16)
    got = np.array([orc.f16_encode(float(x)) for x in xs], np.uint16).view(np.float16)
    assert np.array_equal(ref.view(np.uint16), got.view(np.uint16))


def test_fp16_saturates(orc):
    assert orc.f16_round(1e9) == 65504.0
    assert orc.f16_round(-70000.0) == -65504.0
    assert orc.f16_round(65519.0) == 65504.0


def test_fp16_and_bf16_decode_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = pats.view(np.float16).astype(np.float64)
    refbf = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    for p in range(0, 65536, 13):
        a = orc.f16_decode(p)
        assert (np.isnan(a) and np.isnan(ref16[p])) or a == ref16[p]
        b = orc.bf16_decode(p)
        assert (np.isnan(b) and np.isnan(refbf[p])) or b == refbf[p]


@pytest.mark.parametrize("bits,pb", [(2, 4608), (4, 8704), (3, 0), (8, 0)])
def test_record_bytes(orc, bits, pb):
    assert orc.record_bytes(bits) == pb
