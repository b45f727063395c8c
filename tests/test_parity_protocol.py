"""The comparison protocol accepts the oracle's own records and flags planted
mistakes: it must not excuse real errors as rounding.

Every planted code mistake edits exactly one named code through the documented
record layout (include/kvarn.h, record format 3), and the test first checks,
by unpacking both records, that the edit landed on that (token, channel) and
nowhere else, by the intended number of levels.
"""
import numpy as np
import pytest

import oracle
import parity
from helpers import set_code, tiles_bits
from kv_cache_quantization_x128_amd import synth

META = {2: 2048 * 2, 4: 2048 * 4}   # byte offset of the metadata (s1) per code width


@pytest.fixture(scope="module", params=[(2, 0), (2, 1), (4, 0), (4, 1)], ids=["b2K", "b2V", "b4K", "b4V"])
def case(request):
    bits, axis = request.param
    k, v = synth.tiny()
    view = oracle.TileView.dense(tiles_bits(k if axis == 0 else v)[:3], oracle.DT_F16)
    rec = oracle.quantize(view, bits, axis)
    return view, rec, bits, axis


def test_own_records_pass(case):
    view, rec, bits, axis = case
    rep = parity.compare_quantize(view, bits, axis, rec)
    assert rep["unexplained"] == 0 and rep["raw_identical_codes"] == 1.0


def _plant_code(case, tile, t, c, delta):
    """Copy of the records with the code of (tile, t, c) moved by delta levels;
    asserts that the unpacked records differ exactly there, by delta."""
    view, rec, bits, axis = case
    bad = rec.copy()
    before = oracle.unpack_codes(rec, bits, axis)
    set_code(bad[tile], bits, axis, t, c, int(before[tile, t, c]) + delta)
    after = oracle.unpack_codes(bad, bits, axis)
    d = after.astype(np.int64) - before.astype(np.int64)
    assert np.count_nonzero(d) == 1 and d[tile, t, c] == delta, "the planted edit missed its code"
    return bad


def _decisive(case, tile, max_code):
    """(t, c) of the code of `tile` whose oracle t is farthest from a rounding
    midpoint among codes <= max_code."""
    view, rec, bits, axis = case
    codes, t = oracle.codes_given_meta(view, bits, axis, rec)
    frac = np.abs(np.abs(t[tile] - np.floor(t[tile])) - 0.5)
    frac = np.where(codes[tile] <= max_code, frac, -1.0)
    return np.unravel_index(int(np.argmax(frac)), frac.shape)


def test_code_plus2_is_flagged(case):
    view, rec, bits, axis = case
    t, c = 3, 0                                   # token 3, channel 0 of tile 1
    cur = int(oracle.unpack_codes(rec, bits, axis)[1, t, c])
    delta = 2 if cur + 2 <= 2 ** bits - 1 else -2
    rep = parity.compare_quantize(view, bits, axis, _plant_code(case, 1, t, c, delta))
    assert rep["code_bad"] == 1 and rep["unexplained"] == 1, str(rep)


def test_code_plus1_far_from_tie_is_flagged(case):
    view, rec, bits, axis = case
    t, c = _decisive(case, 0, 2 ** bits - 2)      # the most decisive code that can go up one level
    rep = parity.compare_quantize(view, bits, axis, _plant_code(case, 0, t, c, 1))
    assert rep["code_bad"] == 1 and rep["unexplained"] == 1, str(rep)


def test_code_at_a_tie_is_excused(case):
    """Positive control: the code whose oracle t is closest to k + 1/2, moved to
    the other side of that midpoint, is classed as a tie.  (In each of these
    16384-code tiles the closest t lies within 1e-4 of a midpoint.)"""
    view, rec, bits, axis = case
    codes, t = oracle.codes_given_meta(view, bits, axis, rec)
    frac = np.abs(np.abs(t[2] - np.floor(t[2])) - 0.5)
    ti, ci = np.unravel_index(int(np.argmin(frac)), frac.shape)
    other = int(np.floor(t[2, ti, ci])) if codes[2, ti, ci] == np.floor(t[2, ti, ci]) + 1 else \
        int(np.floor(t[2, ti, ci])) + 1
    delta = other - int(codes[2, ti, ci])
    assert abs(delta) == 1
    rep = parity.compare_quantize(view, bits, axis, _plant_code(case, 2, ti, ci, delta))
    assert frac[ti, ci] <= parity.TIE_ABS
    assert rep["code_ties"] == 1 and rep["unexplained"] == 0, str(rep)


def test_s2_two_steps_is_flagged(case):
    view, rec, bits, axis = case
    bad = rec.copy()
    bad[2, META[bits] + 128 + 10] += 2            # s2 of index 10: two FP8 steps up
    rep = parity.compare_quantize(view, bits, axis, bad)
    assert rep["s2_bad"] >= 1, str(rep)


def test_z_far_is_flagged(case):
    view, rec, bits, axis = case
    bad = rec.copy()
    z = bad[0, META[bits] + 256: META[bits] + 512].view(np.float16).copy()
    z[5] = np.float16(float(z[5]) + 1.0)
    bad[0, META[bits] + 256: META[bits] + 512] = z.view(np.uint8)
    rep = parity.compare_quantize(view, bits, axis, bad)
    assert rep["z_bad"] == 1, str(rep)


def test_s1_swap_is_flagged(case):
    view, rec, bits, axis = case
    bad = rec.copy()
    a, b = META[bits] + 7, META[bits] + 90
    bad[1, a], bad[1, b] = bad[1, b], bad[1, a] + 3
    rep = parity.compare_quantize(view, bits, axis, bad)
    assert rep["s1_bad"] >= 1, str(rep)


def test_many_tile_path_equals_full_protocol():
    """compare_quantize_many (full protocol only for records that differ from the
    oracle's) reports exactly what the full protocol reports, with planted
    mistakes in a few of the tiles and identical records elsewhere."""
    k, _ = synth.tiny()
    tiles = tiles_bits(k)
    rec = oracle.quantize(oracle.TileView.dense(tiles, oracle.DT_F16), 2, 0)
    codes = oracle.unpack_codes(rec, 2, 0)
    bad = rec.copy()
    set_code(bad[1], 2, 0, 3, 0, (int(codes[1, 3, 0]) + 2) % 4)     # a code two levels off
    bad[5, 2048 * 2 + 7] ^= 0x1                                      # an s1 byte one FP8 step off
    set_code(bad[6], 2, 0, 90, 17, (int(codes[6, 90, 17]) + 2) % 4)  # another code
    assert np.count_nonzero(oracle.unpack_codes(bad, 2, 0) != codes) == 2
    full = parity.compare_quantize(oracle.TileView.dense(tiles, oracle.DT_F16), 2, 0, bad)
    many = parity.compare_quantize_many(tiles, oracle.DT_F16, 2, 0, bad, chunk=2)
    assert many["full_protocol_tiles"] == 3
    for key in parity._SUMMED:
        assert many[key] == full[key], key
    assert abs(many["raw_identical_codes"] - full["raw_identical_codes"]) < 1e-15
    assert many["unexplained"] > 0
    same = parity.compare_quantize_many(tiles, oracle.DT_F16, 2, 0, rec)
    assert same["full_protocol_tiles"] == 0 and same["unexplained"] == 0 and same["raw_identical_codes"] == 1.0
