"""GPU parity: decode GEMV and prefill GEMM through the C ABI against the oracle's fp64
accumulation of the dequantized weights (plus fp16 outlier add-back), within the floored
relative tolerance of parity.TOL.  The oracle quantizes the same fp16 weights itself."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu
BITS = (2, 3, 4, 5, 6)


def run_linear(entry, g: GpuWeight, x: np.ndarray, with_csr=True):
    torch, q = gpu()
    m, k = x.shape
    xd = to_dev_fp16(x)
    y = torch.empty((m, g.n), dtype=torch.int16, device="cuda")
    if entry == "qlinear_gemm":
        nnz = g.nnz if with_csr else 0
        wsb = q.qlinear_gemm_workspace_bytes(g.desc, m, nnz)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        q.qlinear_gemm(g.desc, g.handle(with_csr), xd, k, m, y, g.n, ws, wsb)
    else:
        getattr(q, entry)(g.desc, g.handle(with_csr), xd, k, m, y, g.n)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", (1, 3, 8, 16))
def test_gemv_small_with_outliers(bits, m):
    n, k, frac = 64, 1280, 0.002  # 5 k-tiles over 8 waves: idle waves and a ragged split
    w = workloads.weights_fp16(n, k, 300 + bits)
    workloads.plant_outliers(w, frac, 300 + bits)
    x = workloads.activations_fp16(m, k, 300 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac))
    y = run_linear("qlinear_gemv", GpuWeight(w, bits, frac), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("bits", (2, 3, 5, 6, 4))
def test_gemv_layer_4096_full(bits):
    """The single-layer sweep at full size (4096 x 4096), M = 1, 4, 8."""
    w = workloads.layer_weights(1 if bits == 4 else 2)
    ref_q = oracle.quantize(w, bits)
    g = GpuWeight(w, bits)
    for m in (1, 4, 8):
        x = workloads.activations_fp16(m, 4096, workloads.seed_for(2))
        r = oracle.linear(x, ref_q)
        y = run_linear("qlinear_gemv", g, x)
        assert rel_err(y, r) <= TOL, (m, report(y, r))


def test_gemv_one_hot_exact():
    """x = e_k returns fp16(What[:, k]) exactly (a single exact product per output)."""
    n, k = 32, 512
    w = workloads.weights_fp16(n, k, 7)
    qd = oracle.quantize(w, 5)
    g = GpuWeight(w, 5)
    for kstar in (0, 255, 256, 511):
        x = np.zeros((1, k), np.float16)
        x[0, kstar] = 1.0
        r = oracle.linear(x, qd)[0]
        y = run_linear("qlinear_gemv", g, x)[0]
        assert np.array_equal(y, r.astype(np.float16)), kstar


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", (1, 17, 200))
def test_gemm_ragged_with_outliers(bits, m):
    n, k, frac = 560, 1024, 0.002  # n is not a multiple of the 256-row workgroup tile
    w = workloads.weights_fp16(n, k, 400 + bits)
    workloads.plant_outliers(w, frac, 400 + bits)
    x = workloads.activations_fp16(m, k, 400 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac))
    y = run_linear("qlinear_gemm", GpuWeight(w, bits, frac), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("ms,wide", (((1, 1, 1, 1), False), ((1, 1, 1, 1), True), ((1, 3, 8, 2), False),
                                     ((16, 5, 1, 9), True)))
def test_gemv_batch_mixed_bits(ms, wide):
    """Independent problems of different bit widths, shapes and batch sizes (one with
    outliers; `wide` makes the launch large enough for 4-wave workgroups) in one
    qlinear_gemv_batch call."""
    torch, q = gpu()
    specs = [(2, 512, 1024, 0.0), (3, 256, 2048, 0.0), (6, 8192 if wide else 256, 512, 0.0), (4, 384, 1024, 0.004)]
    gws, xs, ys, probs, refs = [], [], [], [], []
    for i, ((bits, n, k, frac), m) in enumerate(zip(specs, ms)):
        w = workloads.weights_fp16(n, k, 700 + i)
        if frac:
            workloads.plant_outliers(w, frac, 700 + i)
        x = workloads.activations_fp16(m, k, 700 + i)
        g = GpuWeight(w, bits, frac)
        xd = to_dev_fp16(x)
        y = torch.empty((m, n), dtype=torch.int16, device="cuda")
        gws.append(g), xs.append(xd), ys.append(y)
        probs.append(q.gemv_problem(g.desc, g.handle(True), xd, k, m, y, n))
        refs.append(oracle.linear(x, oracle.quantize(w, bits, frac)))
    q.qlinear_gemv_batch(probs)
    torch.cuda.synchronize()
    for y, r in zip(ys, refs):
        got = from_dev_fp16(y)
        assert rel_err(got, r) <= TOL, report(got, r)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", (17, 130))
def test_gemm_ragged_dense(bits, m):
    """No outliers: every 16-row activation tile and a partial last weight tile."""
    n, k = 560, 1536
    w = workloads.weights_fp16(n, k, 450 + bits)
    x = workloads.activations_fp16(m, k, 450 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits))
    y = run_linear("qlinear_gemm", GpuWeight(w, bits), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemm_dense_rows_of_outliers():
    """Rows with many outliers (60 in one row, ~20% of ten rows)."""
    n, k, m = 256, 2048, 70
    w = workloads.weights_fp16(n, k, 77)
    rng = np.random.default_rng(77)
    w[3, rng.choice(k, 60, replace=False)] = np.float16(4.0)       # 60 outliers in one row
    w[130:140, :] = np.where(rng.random((10, k)) < 0.2, np.float16(-3.5), w[130:140, :])
    frac = (w.astype(np.float32).__abs__() >= 3).sum() / (n * k)
    frac = (int(round(frac * n * k)) + 0.5) / (n * k)
    x = workloads.activations_fp16(m, k, 77)
    ref = oracle.quantize(w, 4, frac)
    assert len(ref["col"]) > 2048 + 60
    r = oracle.linear(x, ref)
    y = run_linear("qlinear_gemm", GpuWeight(w, 4, frac), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemm_and_gemv_agree():
    w = workloads.weights_fp16(256, 2048, 55)
    x = workloads.activations_fp16(16, 2048, 55)
    g = GpuWeight(w, 4)
    a = run_linear("qlinear_gemv", g, x).astype(np.float64)
    b = run_linear("qlinear_gemm", g, x).astype(np.float64)
    assert rel_err(a, b) <= 2 * TOL


@pytest.mark.timeout(600)
def test_gemm_prefill_full_sampled():
    """M=512, K=8192, N=28672, 4-bit + 0.1% outliers, the shape and launch the benchmark
    times; 512 weight rows (spread over the 112 row tiles) x all 512 activation rows
    recomputed by the oracle."""
    w, pos = workloads.prefill_weights()
    x = workloads.prefill_activations()
    g = GpuWeight(w, 4, workloads.PREFILL_OUTLIER_FRAC)
    y = run_linear("qlinear_gemm", g, x)
    rng = np.random.default_rng(4)
    ns = np.sort(rng.choice(w.shape[0], 512, replace=False))
    ms = np.arange(x.shape[0])
    w0 = w.copy()
    w0.reshape(-1)[pos] = 0
    sub = oracle.quantize(w0[ns], 4)
    # the held-out values of the sampled rows, as an oracle-side CSR
    dense = np.zeros((len(ns), w.shape[1]), np.float16)
    flat_rows, flat_cols = np.divmod(pos, w.shape[1])
    for i, n in enumerate(ns):
        cols = flat_cols[flat_rows == n]
        dense[i, cols] = w[n, cols]
    counts = (dense != 0).sum(1)
    sub["rowptr"] = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rr, cc = np.nonzero(dense)
    sub["col"] = cc.astype(np.int32)
    sub["val"] = dense[rr, cc].view(np.uint16)
    r = oracle.linear(x[ms], sub)
    got = y[np.ix_(ms, ns)]
    assert rel_err(got, r) <= TOL, report(got, r)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("k", (1024, 4096))
def test_gemm_outlier_heavy_rows(k):
    """Rows holding 17, 33 and 40 outliers (the sparse partial's multi-step rows), a weight of
    784 rows (its last 32-row group half full) and m = 70 (one ragged 128-row block of x^T, two
    64-position chunks); k = 4096 also takes the k-split path (the first part seeded)."""
    n, m, frac = 784, 70, 0.004
    w = workloads.weights_fp16(n, k, 4400 + k)
    workloads.plant_outliers(w, 0.003, 4400 + k)
    rng = np.random.default_rng(4401 + k)
    for row, cnt in ((5, 40), (6, 17), (n - 1, 33)):
        cols = rng.choice(k, size=cnt, replace=False)
        w[row, cols] = (rng.uniform(6.0, 8.0, cnt) * rng.choice((-1.0, 1.0), cnt)).astype(np.float16)
    ref_q = oracle.quantize(w, 4, frac)
    counts = np.diff(ref_q["rowptr"])
    assert counts[5] >= 40 and counts[6] >= 17 and counts[n - 1] >= 33, counts[[5, 6, n - 1]]
    x = workloads.activations_fp16(m, k, 4402 + k)
    r = oracle.linear(x, ref_q)
    g = GpuWeight(w, 4, frac)
    assert g.nnz == int(ref_q["rowptr"][-1])
    y = run_linear("qlinear_gemm", g, x)
    assert rel_err(y, r) <= TOL, report(y, r)
