"""Pins of the oracle's codecs against the OCP specifications' own code
tables and rounding rule (fixture: tests/golden/ocp_formats.json) and the
report's 448 x 6 = 2688 bound."""
import json
import os

import numpy as np

from oracle import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ocp_formats.json")))


def test_e2m1_table():
    vals = F.e2m1_value(np.arange(16))
    assert list(vals[:8]) == GOLD["e2m1_positive_values"]
    assert list(vals[8:]) == [-v for v in GOLD["e2m1_positive_values"]]


def test_e4m3fn_points_and_nan():
    for code, v in GOLD["e4m3fn_points"]:
        got = F.e4m3fn_value(int(code, 16))
        assert got == v and np.signbit(got) == np.signbit(v), code
    for code in GOLD["e4m3fn_nan_codes"]:
        assert np.isnan(F.e4m3fn_value(int(code, 16)))
    # strictly increasing over the finite non-negative codes
    pos = F.e4m3fn_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.sum(np.isnan(F.e4m3fn_value(np.arange(256)))) == 2


def test_e8m0_points():
    for code, v in GOLD["e8m0_points"]:
        assert F.e8m0_value(int(code, 16)) == v
    assert np.isnan(F.e8m0_value(0xFF))


def test_page_bound_2688():
    # report section 2.4.4: the format reaches 448 x 6 = 2688
    assert F.e4m3fn_value(0x7E) * F.e2m1_value(0x7) == 2688.0
    assert np.nanmax(F.e4m3fn_value(np.arange(256))) == 448.0
    assert F.e2m1_value(np.arange(16)).max() == 6.0


def test_roundtrip_all_finite_codes():
    c = np.arange(16)
    c = c[c != 8]                       # -0 re-encodes as +0
    assert np.array_equal(F.e2m1_encode(F.e2m1_value(c)), c)
    c = np.arange(256)
    c = c[(c != 0x80) & (c != 0x7F) & (c != 0xFF)]
    assert np.array_equal(F.e4m3fn_encode(F.e4m3fn_value(c)), c)


def test_rne_ties_and_saturation():
    for x, want in GOLD["e2m1_rne_cases"]:
        assert F.e2m1_value(F.e2m1_encode(x)) == want, x
    for x, want in GOLD["e4m3fn_rne_cases"]:
        assert F.e4m3fn_value(F.e4m3fn_encode(x)) == want, x


def test_encode_is_nearest_brute_force():
    # every value's code decodes to a nearest representable value
    rng = np.random.default_rng(0)
    x = rng.uniform(-8, 8, 2000)
    d = np.abs(F.e2m1_value(F.e2m1_encode(x)) - np.clip(x, -6, 6))
    allv = F.e2m1_value(np.arange(16))
    best = np.abs(np.clip(x, -6, 6)[:, None] - allv[None, :]).min(1)
    assert np.allclose(d, best)
    x = np.exp(rng.uniform(np.log(1e-4), np.log(600), 2000))
    allv = F.e4m3fn_value(np.arange(0x7F))
    got = F.e4m3fn_value(F.e4m3fn_encode(x))
    best = np.abs(np.clip(x, 0, 448)[:, None] - allv[None, :]).min(1)
    assert np.allclose(np.abs(got - np.clip(x, 0, 448)), best, rtol=0, atol=0)


def test_nibble_order():
    # channel 2c in the low nibble
    p = F.pack_nibbles(np.array([0x1, 0xA, 0x7, 0x0]))
    assert list(p) == [0xA1, 0x07]
    assert list(F.unpack_nibbles(p)) == [0x1, 0xA, 0x7, 0x0]
