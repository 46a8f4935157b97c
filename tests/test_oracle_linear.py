"""Pins for the oracle's fp64 linear layer y = x * What^T (+ fp16 outlier add-back).

Definition: single-GPU 70B page, s3 (unfused path: dequantize, then matmul(x, W^T)) and
s2 (held-out fp16 weights added back after the GEMM)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def dequant64(q):
    G = q["scales"].shape[1]
    s = q["scales"].view(np.float16).astype(np.float64)
    z = q["zeros"].astype(np.float64)
    return (q["codes"].astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)


def csr_dense(q, N, K):
    d = np.zeros((N, K))
    rows = np.repeat(np.arange(N), np.diff(q["rowptr"]))
    d[rows, q["col"]] = q["val"].view(np.float16).astype(np.float64)
    return d


def test_exact_rational_brute_force():
    """Tiny case: the fp64 result equals the exactly-rounded rational sum to within the
    rounding of a 256-term fp64 sum."""
    M, N, K = 2, 3, 256
    w = workloads.weights_fp16(N, K, 7)
    w[1, 5] = np.float16(4.0)
    x = workloads.activations_fp16(M, K, 7)
    q = oracle.quantize(w, 3, 1.5 / (N * K))
    r = oracle.linear(x, q)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            for k in range(K):
                g = k // 128
                qv = int(q["codes"][n, k]) - int(q["zeros"][n, g])
                s = Fraction(float(np.uint16(q["scales"][n, g]).view(np.float16)))
                exact += Fraction(float(x[m, k])) * qv * s
            for p in range(q["rowptr"][n], q["rowptr"][n + 1]):
                exact += Fraction(float(x[m, q["col"][p]])) * \
                    Fraction(float(np.uint16(q["val"][p]).view(np.float16)))
            assert abs(r[m, n] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))
    assert len(q["col"]) == 1 and q["col"][0] == 5


def test_one_hot_activation_selects_a_weight():
    N, K = 8, 512
    q = oracle.quantize(workloads.weights_fp16(N, K, 11), 5)
    for kstar in (0, 127, 128, 300, 511):
        x = np.zeros((1, K), np.float16)
        x[0, kstar] = 1.0
        assert np.array_equal(oracle.linear(x, q)[0], dequant64(q)[:, kstar])


def test_codes_at_zero_point_leave_only_outliers():
    N, K = 16, 256
    w = np.zeros((N, K), np.float16)
    pos = np.array([3, 700, 2000, 4000])
    w.reshape(-1)[pos] = np.float16([3.5, -4.0, 3.25, 4.75])
    q = oracle.quantize(w, 4, len(pos) / (N * K))
    x = workloads.activations_fp16(3, K, 2)
    want = x.astype(np.float64) @ csr_dense(q, N, K).T
    assert np.array_equal(oracle.linear(x, q), want)
    assert not oracle.linear(x, q, outliers=False).any()


def test_matches_library_matmul():
    """Without rounding-order effects beyond fp64, r equals numpy's fp64 product of x
    with the dequantized weight plus the dense outlier matrix."""
    M, N, K = 4, 48, 1024
    w = workloads.weights_fp16(N, K, 21)
    workloads.plant_outliers(w, 0.002, 21)
    x = workloads.activations_fp16(M, K, 21)
    q = oracle.quantize(w, 6, 0.002)
    want = x.astype(np.float64) @ (dequant64(q) + csr_dense(q, N, K)).T
    got = oracle.linear(x, q)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("g", (32, 64))
def test_small_groups_match_group_routine_and_brute_force(g):
    """Groups of 32 and 64 (mixed-bit page, s2.3: small blocks for the lowest bit widths):
    the matrix quantizer equals the group routine on each g-value group, and the linear
    layer equals a brute-force fp64 product of the dequantized weights."""
    w = workloads.weights_fp16(6, 256, 81)
    for bits, sym in ((2, False), (2, True), (5, False)):
        d = oracle.quantize(w, bits, g=g, sym=sym)
        assert d["scales"].shape == (6, 256 // g) and d["g"] == g
        for n in range(6):
            for j in range(256 // g):
                grp = w[n, g * j: g * (j + 1)]
                if sym:
                    s, q = oracle.quantize_group_sym(grp, bits)
                else:
                    s, z, q = oracle.quantize_group(grp, bits)
                    assert d["zeros"][n, j] == z
                assert d["scales"][n, j] == s
                assert np.array_equal(d["codes"][n, g * j: g * (j + 1)], q)
        x = workloads.activations_fp16(3, 256, 82)
        sc = np.repeat(d["scales"].view(np.float16).astype(np.float64), g, axis=1)
        zp = np.repeat(d["zeros"].astype(np.float64), g, axis=1)
        what = (d["codes"].astype(np.float64) - zp) * sc
        want = x.astype(np.float64) @ what.T
        assert np.allclose(oracle.linear(x, d), want, rtol=1e-12, atol=1e-12)


def test_small_integer_inputs_give_exact_integers():
    """Codes, zero points, power-of-two scales and small-integer activations make every
    dequantized weight and every product a small dyadic number, so the fp64 result must equal
    the integer sum computed in Python's exact integers (no floating point at all), CSR
    outlier terms included."""
    rng = np.random.default_rng(31)
    M, N, K, bits = 3, 32, 512, 5
    G = K // 128
    codes = rng.integers(0, 32, (N, K)).astype(np.uint8)
    zeros = rng.integers(0, 32, (N, G)).astype(np.uint8)
    exps = rng.integers(-2, 3, (N, G))                       # scales 1/4 .. 4
    scales = np.float16(2.0) ** exps.astype(np.float16)
    x = rng.integers(-9, 10, (M, K)).astype(np.float16)
    # three outliers, integer valued, in rows 0, 0 and 17
    rowptr = np.zeros(N + 1, np.int32)
    cols, vals = [5, 400, 77], [3.0, -4.0, 5.0]
    rowptr[1:] = 2
    rowptr[18:] = 3
    q = dict(codes=codes, scales=scales.view(np.uint16), zeros=zeros, rowptr=rowptr,
             col=np.array(cols, np.int32), val=np.array(vals, np.float16).view(np.uint16), g=128)
    r = oracle.linear(x, q)
    xi = x.astype(np.int64)
    for m in range(M):
        for n in range(N):
            acc4 = 0                                       # the sum times 4 (scales >= 1/4)
            for k in range(K):
                g = k // 128
                acc4 += int(xi[m, k]) * (int(codes[n, k]) - int(zeros[n, g])) * (1 << (int(exps[n, g]) + 2))
            for p in range(rowptr[n], rowptr[n + 1]):
                acc4 += 4 * int(xi[m, cols[p]]) * int(vals[p])
            assert r[m, n] * 4 == acc4, (m, n)
    assert np.array_equal(r, np.round(r * 4) / 4)
