"""Pins of the oracle's scalar helpers against numpy and closed forms."""
import math

import numpy as np
import pytest

import oracle


def test_half_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero kept
    assert math.copysign(1.0, oracle.half_to_f64(0x8000)) == -1.0


def test_half_encode_matches_numpy_rne():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(4000) * np.logspace(-9, 5, 4000))
    # exact midpoints between neighbouring halfs (ties go to even) and edges
    for b in [0x0001, 0x03ff, 0x0400, 0x3c00, 0x3c01, 0x7bfe, 0x1234]:
        lo = np.uint16(b).view(np.float16).astype(np.float64)
        hi = np.uint16(b + 1).view(np.float16).astype(np.float64)
        vals += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0), np.nextafter((lo + hi) / 2, 1e9)]
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26]
    got = np.array([oracle.f64_to_half(v) for v in vals], dtype=np.uint16)
    ref = np.array(vals, dtype=np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_silu_closed_forms():
    from scipy.special import expit
    assert oracle.silu(0.0) == 0.0
    for z in [-30.0, -3.5, -1.0, 0.25, 2.0, 17.0]:
        assert oracle.silu(z) == pytest.approx(z * expit(z), rel=1e-14)
    assert oracle.silu(1000.0) == 1000.0
    neg = oracle.silu(-1000.0)
    assert neg == 0.0 and math.copysign(1.0, neg) == -1.0


def test_argmax_lowest_index_on_ties():
    v = np.array([1.0, 5.0, 3.0, 5.0, -2.0])
    i, m = oracle.argmax(v)
    assert i == 1 and m == 0.0
    v = np.array([1.0, 2.0, 7.5, 3.0])
    i, m = oracle.argmax(v)
    assert i == 2 and m == 4.5
