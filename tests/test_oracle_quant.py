"""Pins for the oracle's group quantizer and outlier hold-out.

Formula: inference acceleration guide (mzlw.cn), s1.1: scale = (max-min)/(qmax-qmin),
zero_point = qmin - round(min/scale), q = round(x/scale) + zero_point,
x_hat = (q - zero_point)*scale.  Groups of 128 along K and the top-0.1% |w| held out in
fp16: single-GPU 70B page, s2.  Readings (unsigned codes, RNE, clamping, range extended
to contain 0, fp16 scale floor) are those stated in the oracle's header.

The expected values in the hand-derived cases below were worked out from the formula
by hand (derivation in each comment), not by running any code."""
import numpy as np
import pytest

import oracle
import workloads

H = lambda v: np.float16(v).view(np.uint16).item()


def group(vals, n=128):
    w = np.zeros(n, np.float16)
    w[: len(vals)] = np.array(vals, np.float16)
    return w


def test_all_zero_group():
    s, z, q = oracle.quantize_group(group([]), 4)
    assert (s, z) == (H(1.0), 0) and not q.any()


def test_two_bit_symmetric_range_with_ties():
    # lo=-0.75, hi=0.75 -> s32 = 1.5/3 = 0.5 (exact fp16); zp = -round(-1.5) = 2 (RNE:
    # -1.5 -> -2); q(-0.75) = round(-1.5)+2 = 0; q(0.75) = round(1.5)+2 = 4 -> clamp 3;
    # q(0) = 2.
    s, z, q = oracle.quantize_group(group([-0.75, 0.75]), 2)
    assert s == H(0.5) and z == 2
    assert list(q[:3]) == [0, 3, 2]


def test_three_bit_half_steps_round_to_even():
    # lo=-1.75, hi=1.75 -> s = 3.5/7 = 0.5; zp = -round(-3.5) = 4.
    # x/s:  0.5 -> 0 (even) -> 4;  1.5 -> 2 -> 6;  -0.5 -> -0 -> 4;  -1.5 -> -2 -> 2;
    #       2.5 -> 2 -> 6;  3.5 -> 4 -> 8 -> clamp 7;  -3.5 -> -4 -> 0.
    vals = [0.25, 0.75, -0.25, -0.75, 1.25, 1.75, -1.75]
    s, z, q = oracle.quantize_group(group(vals), 3)
    assert s == H(0.5) and z == 4
    assert list(q[:7]) == [4, 6, 4, 2, 6, 7, 0]


def test_four_bit_inexact_scale():
    # lo=-1, hi=2 -> s32 = 3/15 = 0.2 -> fp16 0x3266 = 0.199951171875;
    # zp = -round(-1/0.19995.. = -5.0012) = 5; q(2) = round(10.0024)+5 = 15;
    # q(-1) = -5+5 = 0; q(0.5) = round(2.5006)+5 = 8.
    s, z, q = oracle.quantize_group(group([-1.0, 2.0, 0.5]), 4)
    assert s == 0x3266 and z == 5
    assert list(q[:4]) == [0, 15, 8, 5]


def test_all_positive_group_keeps_zero_in_range():
    # every weight 1.0: range [0, 1] -> s32 = 1/3 -> fp16 0x3555 = 0.333251953125,
    # zp = 0, q = round(3.0007) = 3.  (With a plain [min, max] range the zero point
    # would be negative and could not be stored in b bits.)
    s, z, q = oracle.quantize_group(np.ones(128, np.float16), 2)
    assert (s, z) == (0x3555, 0) and (q == 3).all()


def test_single_negative_value():
    # [-0.5, 0...] 2-bit: s32 = 0.5/3 -> 0x3155 = 0.1666259765625;
    # zp = -round(-3.0007) = 3; q(-0.5) = 0, q(0) = 3.
    s, z, q = oracle.quantize_group(group([-0.5]), 2)
    assert (s, z) == (0x3155, 3) and q[0] == 0 and (q[1:] == 3).all()


def test_tiny_range_scale_floor():
    # max |w| = 2^-24 (smallest fp16 subnormal): s32 = 2^-24/15 rounds to fp16 zero,
    # so the scale is raised to 2^-14 (0x0400); zp = 0; q = round(2^-10) = 0.
    w = group([])
    w.view(np.uint16)[0] = 1
    s, z, q = oracle.quantize_group(w, 4)
    assert (s, z) == (0x0400, 0) and not q.any()


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_invariants_on_random_groups(bits):
    rng = np.random.default_rng(10 + bits)
    qmax = (1 << bits) - 1
    for trial in range(300):
        std = [0.02, 1.0, 1e-3][trial % 3]
        w = (rng.standard_normal(128) * std + (trial % 5 - 2) * std * 0.7).astype(np.float16)
        s, z, q = oracle.quantize_group(w, bits)
        wf = w.astype(np.float64)
        lo, hi = min(wf.min(), 0.0), max(wf.max(), 0.0)
        sf = np.uint16(s).view(np.float16).astype(np.float64)
        assert 0 <= z <= qmax and q.max() <= qmax
        # fp16 scale is within half an fp16 ulp of the exact (hi-lo)/qmax, or the
        # 2^-14 floor when that quotient is below the smallest normal fp16
        exact = (hi - lo) / qmax
        if exact < 2.0 ** -14:
            assert sf == 2.0 ** -14
        else:
            assert abs(sf - exact) <= exact * 2.0 ** -11 * 1.0001
        # every code reconstructs its weight to within half a step, except where the
        # rounding of the scale pushed the group's extreme past the code range
        err = np.abs(wf - (q.astype(np.float64) - z) * sf)
        clamped = (q == 0) | (q == qmax)
        assert (err[~clamped] <= 0.5 * sf * (1 + 1e-6)).all()
        assert (err <= 0.5 * sf + qmax * abs(sf - exact) + 2 * sf * 1e-6).all()


def test_outliers_recovered_exactly_and_excluded_from_range():
    n, k, frac = 64, 1024, 0.001
    w = workloads.weights_fp16(n, k, 123)
    pos = workloads.plant_outliers(w, frac, 123)
    cnt = oracle.outlier_count(n, k, frac)
    assert cnt == 65 == len(pos)
    r = oracle.quantize(w, 4, frac)
    rows = np.repeat(np.arange(n), np.diff(r["rowptr"]))
    flat = rows.astype(np.int64) * k + r["col"]
    assert np.array_equal(flat, pos)                       # row-major, cols ascending
    assert np.array_equal(r["val"], w.reshape(-1)[pos].view(np.uint16))
    # the held-out slot dequantizes to exactly 0 (its code equals the group's zp)
    g = r["col"] // 128
    assert np.array_equal(r["codes"][rows, r["col"]], r["zeros"][rows, g])
    # the group's scale is the scale of the same group with the outlier set to +0
    w0 = w.copy()
    w0.reshape(-1)[pos] = 0
    r0 = oracle.quantize(w0, 4, 0.0)
    assert np.array_equal(r["scales"], r0["scales"]) and np.array_equal(r["codes"], r0["codes"])


def test_outlier_ties_go_to_lower_index():
    # 40 entries of equal magnitude 1.0 (random signs) but only floor(0.01*16*256) = 40
    # ... make 100 candidates and ask for 40: the first 40 in row-major order win.
    n, k = 16, 256
    w = np.zeros((n, k), np.float16)
    rng = np.random.default_rng(0)
    cand = np.sort(rng.choice(n * k, 100, replace=False))
    w.reshape(-1)[cand] = np.where(rng.integers(0, 2, 100) == 1, 1.0, -1.0)
    frac = 40.5 / (n * k)
    r = oracle.quantize(w, 3, frac)
    rows = np.repeat(np.arange(n), np.diff(r["rowptr"]))
    assert np.array_equal(rows * k + r["col"], cand[:40])


# ---- independent restatement in numpy float32 ---------------------------------------------
#
# The formula of the inference acceleration guide, s1.1, restated with numpy's float32 and
# float16 types under the same readings (range extended to contain 0, RNE via np.rint,
# clamping to [0, qmax], scale stored in fp16 and raised to 2^-14 when it would be zero or
# subnormal, an all-zero group stored as scale 1, zero point 0).  Each numpy float32
# operation is one correctly rounded IEEE operation, and float32 -> float16 is one RNE
# rounding, so this fixes the exact sequence the oracle must follow.  It shares nothing with
# the oracle but the readings.

def np_quantize_groups(w16, bits):
    """[G, n] fp16 groups -> (scale fp16 [G], zero point [G], codes [G, n]) as float arrays."""
    qmax = np.float32((1 << bits) - 1)
    w = w16.astype(np.float32)
    lo = np.minimum(w.min(axis=1), np.float32(0))
    hi = np.maximum(w.max(axis=1), np.float32(0))
    empty = hi == lo
    s32 = (hi - lo) / qmax
    s16 = s32.astype(np.float16)
    s16 = np.where(np.abs(s16) < np.float16(2.0 ** -14), np.float16(2.0 ** -14), s16)
    s16 = np.where(empty, np.float16(1.0), s16)
    sf = s16.astype(np.float32)
    zp = np.clip(np.float32(0) - np.rint(lo / sf), np.float32(0), qmax)
    q = np.clip(np.rint(w / sf[:, None]) + zp[:, None], np.float32(0), qmax)
    zp = np.where(empty, np.float32(0), zp)
    q = np.where(empty[:, None], np.float32(0), q)
    return s16, zp, q


def np_quantize_groups_sym(w16, bits):
    """Symmetric groups (mixed-bit page, s2.3): range [-m, m], implied midpoint zero point."""
    qmax = np.float32((1 << bits) - 1)
    z = np.float32(1 << (bits - 1))
    w = w16.astype(np.float32)
    m = np.abs(w).max(axis=1)
    empty = m == np.float32(0)
    s16 = ((m + m) / qmax).astype(np.float16)
    s16 = np.where(np.abs(s16) < np.float16(2.0 ** -14), np.float16(2.0 ** -14), s16)
    s16 = np.where(empty, np.float16(1.0), s16)
    sf = s16.astype(np.float32)
    q = np.clip(np.rint(w / sf[:, None]) + z, np.float32(0), qmax)
    return s16, q


def random_groups(count, seed):
    """fp16 groups of 128 at three scales, a third of them shifted so the group is one-signed
    or lopsided (the range-contains-zero reading then matters)."""
    rng = np.random.default_rng(seed)
    std = np.array([1e-3, 0.02, 1.0])[rng.integers(0, 3, count)]
    shift = rng.choice([0.0, 0.0, 0.0, 3.0, -3.0, 0.7], count)
    w = rng.standard_normal((count, 128)) * std[:, None] + (shift * std)[:, None]
    return w.astype(np.float16)


def half_step_groups(bits, count, seed):
    """Groups whose values sit exactly on half steps of an exactly representable scale:
    scale 2^e, range [-a*2^e, (qmax-a)*2^e], values (j + 1/2) * 2^e.  Every code is a tie."""
    rng = np.random.default_rng(seed)
    qmax = (1 << bits) - 1
    out = np.zeros((count, 128), np.float16)
    for i in range(count):
        e = int(rng.integers(-12, 2))
        a = int(rng.integers(0, qmax + 1))
        j = rng.integers(-a, qmax - a, 126)
        vals = np.concatenate([[-a, qmax - a], j + 0.5]) * 2.0 ** e
        out[i] = rng.permutation(vals).astype(np.float16)
    return out


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_numpy_float32_restatement_bit_exact(bits):
    """The oracle's quantizer equals the numpy float32 restatement on 10^5 random groups and on
    groups built from exact half steps."""
    w = np.concatenate([random_groups(100_000, 500 + bits), half_step_groups(bits, 2000, 600 + bits)])
    r = oracle.quantize(w, bits)
    s16, zp, q = np_quantize_groups(w, bits)
    assert np.array_equal(r["scales"][:, 0], s16.view(np.uint16))
    assert np.array_equal(r["zeros"][:, 0], zp.astype(np.uint8))
    assert np.array_equal(r["codes"], q.astype(np.uint8))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_numpy_float32_restatement_symmetric(bits):
    w = np.concatenate([random_groups(50_000, 700 + bits), half_step_groups(bits, 1000, 800 + bits)])
    r = oracle.quantize(w, bits, sym=True)
    s16, q = np_quantize_groups_sym(w, bits)
    assert np.array_equal(r["scales"][:, 0], s16.view(np.uint16))
    assert np.array_equal(r["codes"], q.astype(np.uint8))


def test_half_step_groups_are_ties():
    """The tie groups above really put every non-extreme value on a half step of its scale."""
    for bits in (2, 4, 6):
        w = half_step_groups(bits, 50, 900 + bits)
        s16, zp, _ = np_quantize_groups(w, bits)
        t = w.astype(np.float64) / s16.astype(np.float64)[:, None]
        frac = np.abs(t - np.floor(t))
        assert (np.sum(frac == 0.5, axis=1) >= 100).all()


def test_restatement_has_power_against_nearby_mistakes():
    """Three plausible slips in the quantizer each change results on this sample, so the
    bit-exact pins above would catch them: dividing by the fp32 quotient instead of the stored
    fp16 scale, rounding half away from zero instead of to even, and a plain [min, max] range
    instead of one extended to contain 0.  (Forming the scale quotient in double instead of
    fp32 does not change it: a quotient by 2^b - 1 has a repeating bit pattern that cannot
    fall exactly on a binary16 midpoint, so it is not among the slips.)"""
    bits = 3
    w = np.concatenate([random_groups(20_000, 503), half_step_groups(bits, 500, 603)])
    r = oracle.quantize(w, bits)
    qmax = np.float32(7)
    wf = w.astype(np.float32)
    lo = np.minimum(wf.min(axis=1), np.float32(0))
    hi = np.maximum(wf.max(axis=1), np.float32(0))
    s32 = (hi - lo) / qmax
    s32 = np.where(s32 == 0, np.float32(1), s32)
    zp = np.clip(-np.rint(lo / s32), 0, qmax)
    q_unrounded_scale = np.clip(np.rint(wf / s32[:, None]) + zp[:, None], 0, qmax).astype(np.uint8)
    assert np.count_nonzero(q_unrounded_scale != r["codes"]) > 0

    s16, zp16, q16 = np_quantize_groups(w, bits)
    sf = s16.astype(np.float32)[:, None]
    t = wf / sf
    away = np.trunc(t + np.copysign(np.float32(0.5), t))
    q_away = np.clip(away + zp16[:, None], 0, qmax).astype(np.uint8)
    assert np.count_nonzero(q_away != r["codes"]) > 0

    plo, phi = wf.min(axis=1), wf.max(axis=1)
    ps = ((phi - plo) / qmax).astype(np.float16).astype(np.float32)
    ps = np.where(ps == 0, np.float32(1), ps)
    pz = np.clip(-np.rint(plo / ps), 0, qmax)
    q_plain = np.clip(np.rint(wf / ps[:, None]) + pz[:, None], 0, qmax).astype(np.uint8)
    assert np.count_nonzero(q_plain != r["codes"]) > 0
