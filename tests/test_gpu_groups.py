"""GPU parity for groups of 32 and 64 (mixed-bit page, s2.3: small groups for the lowest bit
widths): the quantizer bit for bit against the oracle, and the GEMV and batched GEMV against
the oracle's fp64 products of those weights, within parity.TOL."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16
from test_gpu_matmul import run_linear

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("g", (32, 64))
@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("sym", (False, True))
def test_quantize_bit_exact(g, bits, sym):
    w = workloads.weights_fp16(48, 1280, 950 + bits)
    workloads.plant_outliers(w, 0.002, 950 + bits)
    w[7, 64:128] = 0  # an all-zero group (two at g = 32)
    got = GpuWeight(w, bits, 0.002, sym=sym, g=g).host()
    want = oracle.quantize(w, bits, 0.002, g=g, sym=sym)
    for key in ("codes", "scales", "zeros", "rowptr", "col", "val"):
        assert np.array_equal(got[key], want[key]), key


@pytest.mark.parametrize("g", (32, 64))
@pytest.mark.parametrize("bits", (2, 3, 5, 6))
@pytest.mark.parametrize("m", (1, 8, 16))
def test_gemv_with_outliers(g, bits, m):
    n, k, frac = 64, 1280, 0.002  # 5 k-tiles over 8 waves
    w = workloads.weights_fp16(n, k, 960 + bits)
    workloads.plant_outliers(w, frac, 960 + bits)
    x = workloads.activations_fp16(m, k, 960 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac, g=g))
    y = run_linear("qlinear_gemv", GpuWeight(w, bits, frac, g=g), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("g", (32, 64))
def test_gemv_symmetric_two_bit_wide(g):
    """8192 rows: the 4-wave workgroups; symmetric 2-bit groups, as the page pairs them."""
    w = workloads.weights_fp16(8192, 1024, 970)
    x = workloads.activations_fp16(4, 1024, 971)
    r = oracle.linear(x, oracle.quantize(w, 2, g=g, sym=True))
    y = run_linear("qlinear_gemv", GpuWeight(w, 2, sym=True, g=g), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemv_layer_4096_groups_of_32():
    w = workloads.layer_weights(2)
    g = GpuWeight(w, 2, g=32)
    ref_q = oracle.quantize(w, 2, g=32)
    for m in (1, 8):
        x = workloads.activations_fp16(m, 4096, workloads.seed_for(2))
        y = run_linear("qlinear_gemv", g, x)
        r = oracle.linear(x, ref_q)
        assert rel_err(y, r) <= TOL, (m, report(y, r))


@pytest.mark.parametrize("g", (32, 64))
def test_gemv_batch_one_group_size(g):
    torch, q = gpu()
    specs = [(2, 512, 1024, True), (3, 256, 2048, False), (6, 384, 512, False), (5, 128, 1024, True)]
    keep, ys, probs, refs = [], [], [], []
    for i, (bits, n, k, sym) in enumerate(specs):
        w = workloads.weights_fp16(n, k, 980 + i)
        x = workloads.activations_fp16(3, k, 980 + i)
        gw = GpuWeight(w, bits, sym=sym, g=g)
        xd = to_dev_fp16(x)
        y = torch.empty((3, n), dtype=torch.int16, device="cuda")
        keep.append((gw, xd))
        ys.append(y)
        probs.append(q.gemv_problem(gw.desc, gw.handle(), xd, k, 3, y, n))
        refs.append(oracle.linear(x, oracle.quantize(w, bits, g=g, sym=sym)))
    q.qlinear_gemv_batch(probs)
    torch.cuda.synchronize()
    for y, r in zip(ys, refs):
        got = from_dev_fp16(y)
        assert rel_err(got, r) <= TOL, report(got, r)
