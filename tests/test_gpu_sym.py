"""GPU parity for symmetric groups (implied midpoint zero point, QP_ZERO_MIDPOINT): the
quantizer bit for bit against the oracle's symmetric quantizer, and the GEMV, batched GEMV,
GEMM and grouped GEMM against the oracle's fp64 products of those weights, within
parity.TOL."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16
from test_gpu_matmul import run_linear

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("frac", (0.0, 0.002))
def test_quantize_bit_exact(bits, frac):
    w = workloads.weights_fp16(64, 1280, 900 + bits)
    if frac:
        workloads.plant_outliers(w, frac, 900 + bits)
    w[5, 128:256] = 0  # an all-zero group
    got = GpuWeight(w, bits, frac, sym=True).host()
    want = oracle.quantize(w, bits, frac, sym=True)
    for key in ("codes", "scales", "rowptr", "col", "val"):
        assert np.array_equal(got[key], want[key]), key
    assert (got["codes"][5, 128:256] == 1 << (bits - 1)).all()


@pytest.mark.parametrize("bits", (2, 3, 5))
@pytest.mark.parametrize("m", (1, 8, 16))
def test_gemv_with_outliers(bits, m):
    n, k, frac = 64, 1280, 0.002
    w = workloads.weights_fp16(n, k, 910 + bits)
    workloads.plant_outliers(w, frac, 910 + bits)
    x = workloads.activations_fp16(m, k, 910 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac, sym=True))
    y = run_linear("qlinear_gemv", GpuWeight(w, bits, frac, sym=True), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemv_layer_4096_two_bit():
    w = workloads.layer_weights(2)
    ref_q = oracle.quantize(w, 2, sym=True)
    g = GpuWeight(w, 2, sym=True)
    for m in (1, 8):
        x = workloads.activations_fp16(m, 4096, workloads.seed_for(2))
        y = run_linear("qlinear_gemv", g, x)
        r = oracle.linear(x, ref_q)
        assert rel_err(y, r) <= TOL, (m, report(y, r))


@pytest.mark.parametrize("bits", (2, 3))
@pytest.mark.parametrize("m", (17, 200))
def test_gemm_with_outliers(bits, m):
    n, k, frac = 512, 1024, 0.002
    w = workloads.weights_fp16(n, k, 920 + bits)
    workloads.plant_outliers(w, frac, 920 + bits)
    x = workloads.activations_fp16(m, k, 920 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac, sym=True))
    y = run_linear("qlinear_gemm", GpuWeight(w, bits, frac, sym=True), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemv_batch_mixes_symmetric_and_affine():
    torch, q = gpu()
    specs = [(2, 512, 1024, True), (2, 512, 1024, False), (3, 256, 2048, True), (6, 384, 512, False)]
    keep, ys, probs, refs = [], [], [], []
    for i, (bits, n, k, sym) in enumerate(specs):
        w = workloads.weights_fp16(n, k, 930 + i)
        x = workloads.activations_fp16(4, k, 930 + i)
        g = GpuWeight(w, bits, sym=sym)
        xd = to_dev_fp16(x)
        y = torch.empty((4, n), dtype=torch.int16, device="cuda")
        keep.append((g, xd))
        ys.append(y)
        probs.append(q.gemv_problem(g.desc, g.handle(), xd, k, 4, y, n))
        refs.append(oracle.linear(x, oracle.quantize(w, bits, sym=sym)))
    q.qlinear_gemv_batch(probs)
    torch.cuda.synchronize()
    for y, r in zip(ys, refs):
        got = from_dev_fp16(y)
        assert rel_err(got, r) <= TOL, report(got, r)


@pytest.mark.parametrize("sizes", ([40, 3, 0, 20], [150, 129, 0, 5]), ids=("small-geometry", "layer-geometry"))
def test_grouped_rows(sizes):
    torch, q = gpu()
    E, D, N = len(sizes), 256, 512
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    x = workloads.activations_fp16(R, D, 940)
    raw = [workloads.weights_fp16(N, D, 941 + e) for e in range(E)]
    ws = [GpuWeight(w, 2, sym=True) for w in raw]
    y = torch.empty((R, N), dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ws[0].desc, [w.handle() for w in ws], to_dev_fp16(x), D, None,
                           torch.from_numpy(offsets).cuda(), R, q.QP_EPI_ROWS_F32, y, N)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows):
            r = oracle.linear(x[rows], oracle.quantize(raw[e], 2, sym=True))
            assert rel_err(y[rows], r) <= TOL, (e, report(y[rows], r))
