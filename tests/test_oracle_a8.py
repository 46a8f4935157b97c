"""Pins for the oracle's integer-dot path: dynamic per-token int8 activation quantization
(inference acceleration guide, s1.2: W8A8 quantizes activations to INT8 dynamically per token;
the symmetric INT8 range [-127, 127] of its s1.1 example) and the linear layer on int8
activations times b-bit weights (mixed-bit page, s4.2: integer dot products per group, scale
multiply in floating point).  Hand-derived values are worked out in the comments."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def test_hand_rows():
    # amax 127 -> s = 127/127 = 1 exactly; x/s = x; rint ties to even: -63.5 -> -64, 0.5 -> 0,
    # 1.5 -> 2, -2.5 -> -2.
    x = np.zeros((2, 128), np.float16)
    x[0, :6] = [127, -63.5, 0.5, 1.5, -2.5, 126.5]
    xq, s = oracle.act_quantize(x)
    assert s[0] == 1.0 and list(xq[0, :6]) == [127, -64, 0, 2, -2, 126]
    # all-zero row: scale 0, codes 0
    assert s[1] == 0.0 and not xq[1].any()
    # amax 0.25 -> s = 0.25/127 (fp32); the extreme maps to +-127 exactly, 0.125 to 63.5 of s,
    # which is within an fp32 rounding of the midpoint: check the sign-symmetric pair instead
    y = np.zeros((1, 128), np.float16)
    y[0, :3] = [0.25, -0.25, 0.0]
    q2, s2 = oracle.act_quantize(y)
    assert s2[0] == np.float32(0.25) / np.float32(127) and list(q2[0, :3]) == [127, -127, 0]


def np_act_quantize(x16):
    """Independent numpy float32 restatement."""
    x = x16.astype(np.float32)
    a = np.abs(x).max(axis=1)
    s = a / np.float32(127)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.clip(np.rint(x / s[:, None]), -127, 127)
    q = np.where(a[:, None] == 0, 0, q)
    return q.astype(np.int8), np.where(a == 0, np.float32(0), s).astype(np.float32)


def test_numpy_float32_restatement_bit_exact():
    rng = np.random.default_rng(17)
    rows = []
    for scale in (1e-4, 1e-2, 1.0, 30.0, 1e4):  # finite fp16 inputs (a stated precondition)
        rows.append(np.clip(rng.standard_normal((400, 256)) * scale, -65000, 65000).astype(np.float16))
    ties = np.zeros((50, 256), np.float16)  # rows whose scale is 1: every half-integer is a tie
    ties[:, 0] = 127
    ties[:, 1:] = (rng.integers(-254, 255, (50, 255)) / 2.0).astype(np.float16)
    rows.append(ties)
    x = np.concatenate(rows)
    xq, s = oracle.act_quantize(x)
    q2, s2 = np_act_quantize(x)
    assert np.array_equal(s, s2) and np.array_equal(xq, q2)


def test_layout_map_is_the_stated_piece_order():
    """Inside each 128-k group, 16-byte piece 4*s + t holds k = 64s + 8t .. +7 then
    64s + 32 + 8t .. +7 (s = 64-k step, t = lane quarter)."""
    K = 384
    want = np.empty(K, np.int64)
    for g in range(K // 128):
        for st in range(2):
            for t in range(4):
                piece = g * 128 + 16 * (4 * st + t)
                for e in range(8):
                    want[g * 128 + 64 * st + 8 * t + e] = piece + e
                    want[g * 128 + 64 * st + 32 + 8 * t + e] = piece + 8 + e
    got = np.array([oracle.act_pos(k) for k in range(K)])
    assert np.array_equal(got, want) and np.array_equal(np.sort(got), np.arange(K))
    xq = np.random.default_rng(3).integers(-127, 128, (3, K)).astype(np.int8)
    lay = oracle.act_layout(xq)
    assert np.array_equal(lay[:, want], xq) and np.array_equal(oracle.act_layout(lay, inverse=True), xq)


def test_linear_a8_exact_small_integers():
    """Power-of-two scales: r * 4 / s_x is the exact integer sum, computed in Python integers."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 8, 256
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    zeros = rng.integers(0, 16, (N, K // 128)).astype(np.uint8)
    exps = rng.integers(-2, 3, (N, K // 128))
    q = dict(codes=codes, zeros=zeros, scales=(np.float16(2.0) ** exps.astype(np.float16)).view(np.uint16), g=128)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.array([1.0, 0.5, 0.25], np.float32)
    r = oracle.linear_a8(xq, sx, q)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                isum = sum(int(xq[m, k]) * (int(codes[n, k]) - int(zeros[n, g])) for k in range(128 * g, 128 * g + 128))
                tot += Fraction(2) ** int(exps[n, g]) * isum
            assert Fraction(r[m, n]) == tot * Fraction(float(sx[m]))


def test_linear_a8_against_dequantized_product():
    """Equals the fp64 product of the dequantized activations s_x * xq with the dequantized
    weights (numpy matmul, a different route from the per-group integer sums)."""
    w = workloads.weights_fp16(40, 512, 33)
    q = oracle.quantize(w, 5)
    x = workloads.activations_fp16(6, 512, 34)
    xq, sx = oracle.act_quantize(x)
    G = 4
    wd = (q["codes"].astype(np.float64) - np.repeat(q["zeros"].astype(np.float64), 128, 1)) * \
        np.repeat(q["scales"].view(np.float16).astype(np.float64), 128, 1)
    want = (xq.astype(np.float64) * sx[:, None].astype(np.float64)) @ wd.T
    assert np.allclose(oracle.linear_a8(xq, sx, q), want, rtol=1e-12, atol=1e-12)
