"""GPU parity of the integer-dot path (int8 activations): the per-token activation quantizer
against the oracle's, bit for bit (codes in the library's storage order, fp32 scales), and the
int8-MFMA GEMM against the oracle's fp64 sum of exact integer group dot products, within the
floored relative tolerance of parity.TOL (the GEMM's own error is the fp32 sum over groups and
the one fp16 rounding of y)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu
BITS = (2, 3, 4, 5, 6)


def act_quantize_gpu(x: np.ndarray):
    torch, q = gpu()
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sx = torch.empty(m, dtype=torch.float32, device="cuda")
    q.qact_quantize(to_dev_fp16(x), k, m, k, xq, sx)
    torch.cuda.synchronize()
    return xq, sx


def gemm_a8_gpu(g: GpuWeight, xq, sx, m: int):
    torch, q = gpu()
    y = torch.empty((m, g.n), dtype=torch.int16, device="cuda")
    q.qlinear_gemm_a8(g.desc, g.handle(False), xq, sx, m, y, g.n)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


def special_rows(k: int, seed: int) -> np.ndarray:
    """An all-zero row, a row whose scale is exactly 1 with every half-integer a rounding tie,
    a row with one nonzero value, and rows far from unit scale."""
    rng = np.random.default_rng(seed)
    rows = np.zeros((5, k), np.float16)
    rows[1, 0] = 127
    rows[1, 1:] = (rng.integers(-254, 255, k - 1) / 2.0).astype(np.float16)
    rows[2, k // 3] = -0.75
    rows[3] = (rng.standard_normal(k) * 1e-3).astype(np.float16)
    rows[4] = np.clip(rng.standard_normal(k) * 3e3, -65000, 65000).astype(np.float16)
    return rows


@pytest.mark.parametrize("m,k", ((1, 128), (7, 384), (130, 4096), (300, 1280)))
def test_act_quantize_bit_exact(m, k):
    x = workloads.activations_fp16(m, k, 900 + m)
    x[: min(m, 5)] = special_rows(k, m)[: min(m, 5)]
    xq, sx = act_quantize_gpu(x)
    rq, rs = oracle.act_quantize(x)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oracle.act_layout(rq))


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", (1, 17, 130, 300))
def test_gemm_a8_ragged(bits, m):
    """Every bit width; a partial last weight tile (n = 560); one partial 256-row activation
    block, or a full one and a partial one (m = 300)."""
    n, k = 560, 1536
    w = workloads.weights_fp16(n, k, 950 + bits)
    x = workloads.activations_fp16(m, k, 950 + bits)
    if m > 5:
        x[:5] = special_rows(k, bits)
    xq, sx = act_quantize_gpu(x)
    rq, rs = oracle.act_quantize(x)
    r = oracle.linear_a8(rq, rs, oracle.quantize(w, bits))
    y = gemm_a8_gpu(GpuWeight(w, bits), xq, sx, m)
    assert rel_err(y, r) <= TOL, report(y, r)
    if m > 5:
        assert not y[0].any()  # the all-zero row: scale 0


@pytest.mark.parametrize("bits", (2, 3, 4))
def test_gemm_a8_symmetric(bits):
    """Implied midpoint zero points (none stored)."""
    n, k, m = 256, 1024, 64
    w = workloads.weights_fp16(n, k, 970 + bits)
    x = workloads.activations_fp16(m, k, 970 + bits)
    xq, sx = act_quantize_gpu(x)
    rq, rs = oracle.act_quantize(x)
    r = oracle.linear_a8(rq, rs, oracle.quantize(w, bits, sym=True))
    y = gemm_a8_gpu(GpuWeight(w, bits, sym=True), xq, sx, m)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemm_a8_integer_exact():
    """Small integer weights and activations whose every result is an exact fp16 integer:
    amax 127 gives s_x = 1, so xq = x; the weight rows are quantized exactly by the oracle
    (scale 1, zero point the row minimum).  y must equal the integer product bit for bit."""
    n, k, m = 32, 256, 16
    rng = np.random.default_rng(5)
    w = rng.integers(-7, 9, (n, k)).astype(np.float16)
    w[:, 0], w[:, 1] = -7, 8                     # every group spans [-7, 8]: scale 1 at 4 bits
    w[:, 128], w[:, 129] = -7, 8
    x = rng.integers(-3, 4, (m, k)).astype(np.float16)
    x[:, 5] = 127                                # s_x = 1
    qd = oracle.quantize(w, 4)
    assert np.all(qd["scales"].view(np.float16) == 1)
    xq, sx = act_quantize_gpu(x)
    exact = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.abs(exact).max() < 2048
    y = gemm_a8_gpu(GpuWeight(w, 4), xq, sx, m)
    assert np.array_equal(y.astype(np.int64), exact)


@pytest.mark.timeout(600)
def test_gemm_a8_prefill_full_sampled():
    """M=512, K=8192, N=28672, 4-bit g=128, the shape and launch the benchmark times (no
    outliers held out: they are quantized in their groups); 512 weight rows spread over the 112
    row tiles x all 512 activation rows recomputed by the oracle."""
    w, _ = workloads.prefill_weights()
    x = workloads.prefill_activations()
    g = GpuWeight(w, 4)
    xq, sx = act_quantize_gpu(x)
    rq, rs = oracle.act_quantize(x)
    assert np.array_equal(xq.cpu().numpy(), oracle.act_layout(rq))
    y = gemm_a8_gpu(g, xq, sx, x.shape[0])
    ns = np.sort(np.random.default_rng(8).choice(w.shape[0], 512, replace=False))
    r = oracle.linear_a8(rq, rs, oracle.quantize(w[ns], 4))
    got = y[:, ns]
    assert rel_err(got, r) <= TOL, report(got, r)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("sym", (False, True))
def test_gemm_a8_fp8_scales(bits, sym):
    """fp8 group scales with fallback groups on int8 activations: the integer group sums
    scaled by the E4M3 values (or the fallback's fp16 scale) and the row factor, against the
    oracle's integer-dot product over the same weights; a partial last weight tile and a
    ragged activation block."""
    from test_gpu_fp8 import GpuWeightFp8, plant_fallbacks
    torch, q = gpu()
    n, k, m = 560, 1536, 130
    w = workloads.weights_fp16(n, k, 960 + bits)
    plant_fallbacks(w, 128, 960 + bits, rows=(0, 300, 559))
    x = workloads.activations_fp16(m, k, 961 + bits)
    xq, sx = act_quantize_gpu(x)
    rq, rs = oracle.act_quantize(x)
    qd = oracle.quantize_fp8(w, bits, 128, sym=sym)
    assert qd["counts"][300] == 3
    g = GpuWeightFp8(w, bits, 128, sym)
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    q.qlinear_gemm_a8(g.desc, g.handle(), xq, sx, m, y, n)
    torch.cuda.synchronize()
    got = from_dev_fp16(y)
    r = oracle.linear_a8_fp8(rq, rs, qd)
    assert rel_err(got, r) <= TOL, report(got, r)
