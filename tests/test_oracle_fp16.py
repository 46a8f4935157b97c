"""Pins for the oracle's IEEE binary16 conversions.

The oracle's fp16 rounding is a plain restatement of IEEE 754 round-to-nearest-even;
numpy's float64 -> float16 cast implements the same rounding, so on these inputs the
two must agree bit for bit (a special case that reduces to a library routine)."""
import numpy as np

import oracle


def test_half_value_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_value(int(p)) for p in pats[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(r) & (r > 0))


def test_round_half_matches_ieee_rne():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        rng.uniform(-70000, 70000, 500),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0, -1.0]),
    ])
    # exact ties between neighbouring fp16 values: RNE must pick the even one
    h = rng.integers(0x0001, 0x7BFF, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, (lo + hi) / 2, -(lo + hi) / 2])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.round_half(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
