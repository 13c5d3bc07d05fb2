"""Pins of the oracle's fp16 <-> fp32 conversions against numpy's IEEE binary16
conversions (a library routine; round to nearest even)."""
import numpy as np

import oracle


def test_half_to_float_all_patterns():
    lib = oracle._load()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([lib.orc_half_to_float(int(h)) for h in pats], dtype=np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def _check_to_half(vals):
    lib = oracle._load()
    vals = np.asarray(vals, dtype=np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([lib.orc_float_to_half(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_float_to_half_exact_values():
    pats = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # all finite non-negative fp16
    v = pats.view(np.float16).astype(np.float32)
    _check_to_half(np.concatenate([v, -v]))


def test_float_to_half_ties_and_neighbours():
    # midpoints between consecutive fp16 values are exact fp32 numbers: ties must go to even
    pats = np.arange(0, 0x7BFF, dtype=np.uint32).astype(np.uint16)
    a = pats.view(np.float16).astype(np.float64)
    b = (pats + 1).view(np.float16).astype(np.float64)
    mid = ((a + b) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    _check_to_half(np.concatenate([mid, up, dn, -mid]))


def test_float_to_half_overflow_and_random():
    edge = np.array([65504, 65519.996, 65520, 65536, 1e6, 3e38, np.inf, 2.0**-24, 2.0**-25,
                     1.5 * 2.0**-25, 2.0**-26, 0.0, -0.0, 2.0**-14, np.nextafter(2.0**-14, 0)],
                    dtype=np.float32)
    _check_to_half(edge)
    rng = np.random.default_rng(1)
    r = (rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 17, 20000))).astype(np.float32)
    _check_to_half(r)
