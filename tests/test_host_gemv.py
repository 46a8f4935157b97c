"""Host fused unpack + multiply-accumulate GEMV (qlinear_gemv_host, the CPU half of a CPU/GPU
layer split, mixed-bit page s4.1/s4.3) against the oracle's fp64 linear layer, within the
floored relative tolerance of the GPU matmuls: every width, group sizes 128/64/32, byte and
implied zero points, 1-8 activation rows, outliers, ragged row counts, and each of the three
paths (AVX-512 with byte permutes where the host has it, AVX2, portable).  CPU only."""
import os

import numpy as np
import pytest

import oracle
import weight_only_mixed_amd as q
import workloads
from parity import TOL, rel_err, report


def run_host(w, bits, x, g=128, sym=False, frac=0.0, threads=0):
    n, k = w.shape
    m = x.shape[0]
    r = oracle.quantize(w, bits, frac, g=g, sym=sym)
    packed = np.ascontiguousarray(oracle.pack_canonical(r["codes"], bits))
    scales = np.ascontiguousarray(r["scales"])
    zeros = np.ascontiguousarray(r["zeros"])
    rowptr, col, val = (np.ascontiguousarray(r["rowptr"], np.int32), np.ascontiguousarray(r["col"], np.int32),
                        np.ascontiguousarray(r["val"], np.uint16))
    nnz = len(col)
    wh = q.qp_weight(packed.ctypes.data, scales.ctypes.data, None if sym else zeros.ctypes.data,
                     rowptr.ctypes.data if nnz else None, col.ctypes.data if nnz else None,
                     val.ctypes.data if nnz else None, nnz)
    d = q.desc(bits, n, k, q.QP_LAYOUT_CANONICAL, group_size=g,
               zero_mode=q.QP_ZERO_MIDPOINT if sym else q.QP_ZERO_STORED)
    xs = np.ascontiguousarray(x).view(np.uint16)
    y = np.zeros((m, n), np.uint16)
    q.qlinear_gemv_host(d, wh, xs, k, m, y, n, threads)
    return y.view(np.float16).astype(np.float64), oracle.linear(x, r)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("m", (1, 2, 3, 8))
def test_widths_and_rows_with_outliers(bits, m):
    n, k = 70, 1024  # 70 rows: tiles of 4 and 2 rows plus remainders
    w = workloads.weights_fp16(n, k, 900 + bits)
    workloads.plant_outliers(w, 0.003, 900 + bits)
    x = workloads.activations_fp16(m, k, 901 + bits)
    y, r = run_host(w, bits, x, frac=0.003)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("g,sym,bits", [(64, False, 5), (32, False, 2), (32, True, 2), (64, True, 3), (128, True, 4)])
def test_group_sizes_and_implied_zero_points(g, sym, bits):
    w = workloads.weights_fp16(48, 512, 910)
    x = workloads.activations_fp16(4, 512, 911)
    y, r = run_host(w, bits, x, g=g, sym=sym)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_full_layer_4096_and_thread_counts():
    w = workloads.layer_weights(1)
    x = workloads.activations_fp16(1, 4096, workloads.seed_for(1))
    y1, r = run_host(w, 4, x, threads=1)
    assert rel_err(y1, r) <= TOL, report(y1, r)
    y0, _ = run_host(w, 4, x, threads=0)
    assert np.array_equal(y0, y1)  # rows are independent: the thread count changes nothing


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_avx2_path(monkeypatch, bits):
    monkeypatch.setenv("QPACK_HOST_AVX2", "1")
    w = workloads.weights_fp16(36, 512, 930 + bits)
    workloads.plant_outliers(w, 0.004, 930 + bits)
    x = workloads.activations_fp16(3, 512, 931)
    y, r = run_host(w, bits, x, g=64 if bits == 5 else 128, frac=0.004)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_path_query(monkeypatch):
    monkeypatch.delenv("QPACK_HOST_AVX2", raising=False)
    monkeypatch.delenv("QPACK_HOST_PORTABLE", raising=False)
    best = q.qlinear_gemv_host_isa()
    assert best in ("avx512vbmi", "avx2", "portable")
    monkeypatch.setenv("QPACK_HOST_AVX2", "1")
    assert q.qlinear_gemv_host_isa() == ("portable" if best == "portable" else "avx2")
    monkeypatch.setenv("QPACK_HOST_PORTABLE", "1")
    assert q.qlinear_gemv_host_isa() == "portable"


def test_portable_path(monkeypatch):
    monkeypatch.setenv("QPACK_HOST_PORTABLE", "1")
    for bits in (3, 6):
        w = workloads.weights_fp16(40, 512, 920 + bits)
        workloads.plant_outliers(w, 0.004, 920 + bits)
        x = workloads.activations_fp16(2, 512, 921)
        y, r = run_host(w, bits, x, frac=0.004)
        assert rel_err(y, r) <= TOL, report(y, r)


def test_rejections():
    d = q.desc(4, 64, 512, q.QP_LAYOUT_DEVICE)
    z = np.zeros(64 * 512, np.uint8)
    wh = q.qp_weight(z.ctypes.data, z.ctypes.data, z.ctypes.data, None, None, None, 0)
    x = np.zeros((9, 512), np.uint16)
    y = np.zeros((9, 64), np.uint16)
    assert q.qlinear_gemv_host(d, wh, x, 512, 1, y, 64, check=False) == q.QP_ERR_UNSUPPORTED  # device layout
    d = q.desc(4, 64, 512, q.QP_LAYOUT_CANONICAL)
    assert q.qlinear_gemv_host(d, wh, x, 512, 9, y, 64, check=False) == q.QP_ERR_UNSUPPORTED  # m > 8
    assert q.qlinear_gemv_host(d, wh, x, 500, 1, y, 64, check=False) == q.QP_ERR_INVALID_ARG  # ldx < k


def shrink_groups(w: np.ndarray, g: int, row: int, groups):
    """Scale groups of one row by 2^-16: they fall outside E4M3's range below the row's
    largest scale and take fp16 fallback scales."""
    for c in groups:
        w[row, c * g:(c + 1) * g] = (w[row, c * g:(c + 1) * g].astype(np.float32) * 2.0 ** -16).astype(np.float16)


def run_host_fp8(w, bits, x, g, sym, fb_stride=8):
    n, k = w.shape
    m = x.shape[0]
    qd = oracle.quantize_fp8(w, bits, g, sym=sym, fb_stride=fb_stride)
    packed = np.ascontiguousarray(oracle.pack_canonical(qd["codes"], bits))
    sc8, fac = np.ascontiguousarray(qd["sc8"]), np.ascontiguousarray(qd["factors"])
    fb = np.ascontiguousarray(qd["fb"]) if fb_stride else None
    zeros = None if sym else np.ascontiguousarray(qd["zeros"])
    wh = q.weight_fp8(packed.ctypes.data, sc8.ctypes.data, fac.ctypes.data, fb.ctypes.data if fb is not None else None,
                      fb_stride, zeros.ctypes.data if zeros is not None else None)
    d = q.desc(bits, n, k, q.QP_LAYOUT_CANONICAL, group_size=g,
               zero_mode=q.QP_ZERO_MIDPOINT if sym else q.QP_ZERO_STORED, scale_format=q.QP_SCALE_FP8)
    y = np.zeros((m, n), np.uint16)
    q.qlinear_gemv_host(d, wh, np.ascontiguousarray(x).view(np.uint16), k, m, y, n, 0)
    return y.view(np.float16).astype(np.float64), oracle.linear_fp8(x, qd), qd


@pytest.mark.parametrize("path", ("best", "avx2", "portable"))
@pytest.mark.parametrize("bits,g,sym", ((2, 32, True), (3, 64, False), (4, 128, False), (5, 32, True), (6, 64, False)))
def test_fp8_scales(monkeypatch, path, bits, g, sym):
    """fp8 scales with fallback groups on every path: each group's scale is the row factor
    times its E4M3 value, or its fp16 fallback."""
    monkeypatch.delenv("QPACK_HOST_AVX2", raising=False)
    monkeypatch.delenv("QPACK_HOST_PORTABLE", raising=False)
    if path == "avx2":
        monkeypatch.setenv("QPACK_HOST_AVX2", "1")
    elif path == "portable":
        monkeypatch.setenv("QPACK_HOST_PORTABLE", "1")
    w = workloads.weights_fp16(40, 512, 940 + bits)
    shrink_groups(w, g, 0, (1, 3))
    shrink_groups(w, g, 21, (0,))
    x = workloads.activations_fp16(3, 512, 941)
    y, r, qd = run_host_fp8(w, bits, x, g, sym)
    assert qd["counts"][0] == 2 and qd["counts"][21] == 1
    assert rel_err(y, r) <= TOL, report(y, r)


def test_fp8_fallback_index_past_the_list():
    """More fallback groups than slots: bytes naming a slot past the list read its last slot
    (as the GPU paths do); without a list they read scale 0."""
    g, k = 32, 512
    w = workloads.weights_fp16(16, k, 950, std=0.002)
    w[5, :g] = workloads.weights_fp16(1, g, 951, std=100.0)  # row 5: 15 fallbacks
    x = workloads.activations_fp16(2, k, 952)
    x[:, :g] = 0
    y, _, qd = run_host_fp8(w, 4, x, g, False, fb_stride=4)
    assert qd["counts"][5] == k // g - 1
    sc = qd["scales_f32"].copy()
    last = np.float32(oracle.half_value(int(qd["fb"][5, 3])))
    for gi in range(k // g):
        b = int(qd["sc8"][5, gi])
        if b & 0x80 and (b & 0x7F) >= 4:
            sc[5, gi] = last
    r = oracle.linear_fp8(x, dict(qd, scales_f32=sc))
    assert rel_err(y, r) <= TOL, report(y, r)
