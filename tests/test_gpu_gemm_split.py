"""GPU parity of the k-split prefill GEMM (shapes whose 256 x 128 output tiles fill at most half
of the CUs: k cut into 2, 4 or 8 parts of fp32 partial rows, summed in part order with the
outlier partial before the one fp16 rounding) against the oracle, and against the same call
without the split's workspace; the TP = 8 shard of the prefill case (N = 3584) on sampled rows."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu


def gemm(g, x, split: bool, with_csr: bool = True, fp8: bool = False):
    torch, q = gpu()
    m, k = x.shape
    y = torch.empty((m, g.n), dtype=torch.int16, device="cuda")
    h = g.handle() if fp8 else g.handle(with_csr)
    nnz = 0 if fp8 or not with_csr else g.nnz
    wsb = q.qlinear_gemm_workspace_bytes(g.desc, m, nnz)
    if not split:  # only the outlier part: the GEMM runs unsplit
        wsb = 0
        if nnz:
            ldt = (m + 127) // 128 * 128
            wsb = (2 * g.k + 4 * g.n) * ldt
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    q.qlinear_gemm(g.desc, h, to_dev_fp16(x), k, m, y, g.n, ws if wsb else None, wsb)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


def split_parts(q, d, m) -> int:
    """Parts the library will use: the workspace beyond the outlier part, in m x n fp32 planes."""
    return q.qlinear_gemm_workspace_bytes(d, m, 0) // (4 * m * d.n)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("m", (64, 200))
def test_split_dense_every_width(bits, m):
    """n = 512, k = 4096: 2 (m = 64) or 4 (m = 200, one full and one ragged row tile) output
    tiles, so k splits 8 ways; split and unsplit both against the oracle."""
    torch, q = gpu()
    n, k = 512, 4096
    w = workloads.weights_fp16(n, k, 5000 + bits)
    x = workloads.activations_fp16(m, k, 5001 + bits)
    g = GpuWeight(w, bits)
    assert split_parts(q, g.desc, m) == 8
    r = oracle.linear(x, oracle.quantize(w, bits))
    ys, yu = gemm(g, x, True), gemm(g, x, False)
    assert rel_err(ys, r) <= TOL, report(ys, r)
    assert rel_err(yu, r) <= TOL, report(yu, r)


@pytest.mark.parametrize("g_,sym,packed", ((32, True, False), (64, False, True), (128, False, True), (32, False, False)))
def test_split_metadata_variants(g_, sym, packed):
    """Groups of 32 / 64, implied and b-bit zero points through the split."""
    n, k, m = 256, 2048, 96
    w = workloads.weights_fp16(n, k, 5100 + g_)
    x = workloads.activations_fp16(m, k, 5101)
    g = GpuWeight(w, 3, g=g_, sym=sym, packed_zeros=packed)
    r = oracle.linear(x, oracle.quantize(w, 3, g=g_, sym=sym))
    y = gemm(g, x, True)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("m", (70, 129))
def test_split_with_outliers(m):
    """The outlier partial (S^T, in its transposed row order) is added in the reduction."""
    n, k = 768, 4096
    w = workloads.weights_fp16(n, k, 5200)
    workloads.plant_outliers(w, 0.002, 5200)
    x = workloads.activations_fp16(m, k, 5201)
    g = GpuWeight(w, 4, 0.002)
    assert g.nnz > 0
    r = oracle.linear(x, oracle.quantize(w, 4, 0.002))
    ys, yu = gemm(g, x, True), gemm(g, x, False)
    assert rel_err(ys, r) <= TOL, report(ys, r)
    assert rel_err(yu, r) <= TOL, report(yu, r)


def test_split_fp8_scales():
    from test_gpu_fp8 import GpuWeightFp8, plant_fallbacks
    n, k, m = 512, 4096, 100
    w = workloads.weights_fp16(n, k, 5300)
    plant_fallbacks(w, 32, 5300, rows=(0, 300, 511))
    x = workloads.activations_fp16(m, k, 5301)
    g = GpuWeightFp8(w, 2, 32, True)
    r = oracle.linear_fp8(x, oracle.quantize_fp8(w, 2, 32, sym=True))
    y = gemm(g, x, True, fp8=True)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.timeout(600)
def test_split_prefill_tp8_shard_sampled():
    """The prefill case's TP = 8 shard: M = 512, K = 8192, N = 3584 (the first 3584 rows of its
    weight, 4-bit, 0.1% outliers): 56 output tiles, k split 4 ways; 256 weight rows x all 512
    activation rows recomputed by the oracle."""
    torch, q = gpu()
    w, _ = workloads.prefill_weights()
    w = np.ascontiguousarray(w[:3584])
    x = workloads.prefill_activations()
    g = GpuWeight(w, 4, workloads.PREFILL_OUTLIER_FRAC)
    assert split_parts(q, g.desc, 512) == 4
    y = gemm(g, x, True)
    ns = np.sort(np.random.default_rng(6).choice(3584, 256, replace=False))
    ref = oracle.quantize(w, 4, workloads.PREFILL_OUTLIER_FRAC)
    sub = dict(codes=ref["codes"][ns], scales=ref["scales"][ns], zeros=ref["zeros"][ns])
    rp = ref["rowptr"]
    cols, vals, ptr = [], [], [0]
    for n_ in ns:
        cols.append(ref["col"][rp[n_]:rp[n_ + 1]])
        vals.append(ref["val"][rp[n_]:rp[n_ + 1]])
        ptr.append(ptr[-1] + rp[n_ + 1] - rp[n_])
    sub["rowptr"] = np.array(ptr, np.int32)
    sub["col"] = np.concatenate(cols).astype(np.int32)
    sub["val"] = np.concatenate(vals).astype(np.uint16)
    r = oracle.linear(x, sub)
    got = y[:, ns]
    assert rel_err(got, r) <= TOL, report(got, r)
