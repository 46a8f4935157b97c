"""Pins for the oracle's symmetric group quantizer.

Mixed-bit page (pwwt.cn), s2.3: at 2 and 3 bits the zero point is dropped and the
block's scale absorbs the offset.  Reading (stated in the oracle's header): the group
range is [-m, m] with m = max |w|, so scale = fp16((m + m) / qmax) and the zero point is
the midpoint 2^(b-1) -- what the affine formula of the inference acceleration guide
(mzlw.cn, s1.1) gives for that range -- implied rather than stored; codes are
clamp(round(w/scale) + 2^(b-1), 0, qmax) with round-half-to-even.

The expected values in the hand-derived cases were worked out from these formulas by
hand (derivation in each comment), not by running any code."""
import numpy as np
import pytest

import oracle
import workloads

H = lambda v: np.float16(v).view(np.uint16).item()


def group(vals, n=128):
    w = np.zeros(n, np.float16)
    w[: len(vals)] = np.array(vals, np.float16)
    return w


@pytest.mark.parametrize("bits", (2, 3, 6))
def test_all_zero_group_sits_at_the_midpoint(bits):
    s, q = oracle.quantize_group_sym(group([]), bits)
    assert s == H(1.0) and (q == 1 << (bits - 1)).all()


def test_two_bit_exact_scale_with_ties():
    # m = 1.5 -> (1.5 + 1.5) / 3 = 1.0; z = 2.  1.5 -> round(1.5) = 2 (RNE) -> 4 -> clamp 3;
    # -1.5 -> -2 -> 0; 0.75 -> 1 -> 3; 0.5 -> 0 (RNE) -> 2; 0 -> 2.
    s, q = oracle.quantize_group_sym(group([1.5, -1.5, 0.75, 0.5]), 2)
    assert s == H(1.0)
    assert list(q[:5]) == [3, 0, 3, 2, 2]


def test_three_bit_exact_scale_with_ties():
    # m = 3.5 -> 7 / 7 = 1.0; z = 4.  3.5 -> 4 (RNE) -> 8 -> clamp 7; -3.5 -> -4 -> 0;
    # 2.5 -> 2 (RNE) -> 6; -0.5 -> -0 -> 4; 1.375 -> 1 -> 5.
    s, q = oracle.quantize_group_sym(group([3.5, -3.5, 2.5, -0.5, 1.375]), 3)
    assert s == H(1.0)
    assert list(q[:5]) == [7, 0, 6, 4, 5]


def test_two_bit_inexact_scale():
    # m = 1 -> 2/3 = 0.10101010101|0101... (binary) -> fp16 rounds down to
    # 0.66650390625 (0x3955).  1/0.6665... = 1.50037 -> 2 -> clamp 3; -1 -> -2 -> 0;
    # fp16(1/3) = 0.333251953125 is exactly half the scale -> 0 (RNE) -> 2, same for its
    # negative; 0.99951171875 / 0.66650390625 = 1.49963 -> 1 -> 3.
    s, q = oracle.quantize_group_sym(group([1.0, -1.0, 0.333251953125, -0.333251953125, 0.99951171875]), 2)
    assert s == 0x3955
    assert list(q[:5]) == [3, 0, 2, 2, 3]


def test_tiny_range_scale_floor():
    # m = 2^-20: 2m/3 is far below the smallest normal fp16, so the scale is 2^-14 and
    # every weight rounds to the midpoint.
    s, q = oracle.quantize_group_sym(group([2.0 ** -20, -(2.0 ** -20)]), 2)
    assert s == 0x0400 and (q == 2).all()


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_invariants_on_random_groups(bits):
    rng = np.random.default_rng(40 + bits)
    qmax, z = (1 << bits) - 1, 1 << (bits - 1)
    for trial in range(300):
        std = [0.02, 1.0, 1e-3][trial % 3]
        w = (rng.standard_normal(128) * std + (trial % 5 - 2) * std * 0.7).astype(np.float16)
        s, q = oracle.quantize_group_sym(w, bits)
        wf = w.astype(np.float64)
        m = np.abs(wf).max()
        sf = np.uint16(s).view(np.float16).astype(np.float64)
        assert q.max() <= qmax
        exact = 2 * m / qmax
        if exact < 2.0 ** -14:
            assert sf == 2.0 ** -14
        else:
            assert abs(sf - exact) <= exact * 2.0 ** -11 * 1.0001
        err = np.abs(wf - (q.astype(np.float64) - z) * sf)
        # below the top code every weight is within half a step (no weight in [-m, m] is
        # clamped at code 0: that needs |w| > (z + 1/2) scale, about m (2^b + 1) / (2^b - 1))
        top = q == qmax
        assert (err[~top] <= 0.5 * sf * (1 + 1e-6)).all()
        # at the top code: w - (qmax - z) scale <= scale/2 + (qmax/2) |scale - exact|
        assert (err <= 0.5 * sf + 0.5 * qmax * abs(sf - exact) + 2 * sf * 1e-6).all()


@pytest.mark.parametrize("bits", (2, 3, 5))
def test_agrees_with_asymmetric_on_symmetric_data(bits):
    # For a group holding both m and -m the affine quantizer sees the range [-m, m]: the
    # same scale, and where its rounded zero point is the midpoint, the same codes.
    rng = np.random.default_rng(60 + bits)
    z = 1 << (bits - 1)
    same = 0
    for trial in range(200):
        half = (rng.standard_normal(64) * 0.02).astype(np.float16)
        w = np.concatenate([half, -half])
        rng.shuffle(w)
        s_a, z_a, q_a = oracle.quantize_group(w, bits)
        s_s, q_s = oracle.quantize_group_sym(w, bits)
        assert s_a == s_s
        if z_a == z:
            assert np.array_equal(q_a, q_s)
            same += 1
    assert same > 50


def test_matrix_quantize_with_outliers_matches_groups():
    w = workloads.weights_fp16(8, 256, 71)
    w[3, 17] = np.float16(4.0)
    w[5, 200] = np.float16(-3.5)
    d = oracle.quantize(w, 2, outlier_frac=2 / (8 * 256), sym=True)
    assert d["sym"] and (d["zeros"] == 2).all()
    assert list(zip(np.repeat(np.arange(8), np.diff(d["rowptr"])), d["col"])) == [(3, 17), (5, 200)]
    for n in range(8):
        for g in range(2):
            grp = w[n, 128 * g: 128 * (g + 1)].copy()
            if (n, g) == (3, 0):
                grp[17] = 0
            if (n, g) == (5, 1):
                grp[72] = 0
            s, q = oracle.quantize_group_sym(grp, 2)
            assert d["scales"][n, g] == s
            assert np.array_equal(d["codes"][n, 128 * g: 128 * (g + 1)], q)
