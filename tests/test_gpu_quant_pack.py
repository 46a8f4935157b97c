"""GPU parity: quantize, pack and unpack through the C ABI must match the CPU oracle
bit for bit (integer and byte work)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import GpuWeight, gpu

pytestmark = pytest.mark.gpu
BITS = (2, 3, 4, 5, 6)


def edge_matrix(n, k, seed):
    """N(0, 0.02) weights plus hand-made degenerate groups in the first rows."""
    w = workloads.weights_fp16(n, k, seed)
    w[0, 0:128] = 0                                  # all-zero group
    w[0, 128:256] = np.float16(0.125)                # constant positive group
    w[1, 0:128] = np.float16(-0.5)                   # constant negative group
    w[1, 128:256] = 0
    w[1, 130] = np.float16(-0.75)                    # exact ties at half steps
    w[1, 131] = np.float16(0.75)
    w[2, 0:128] = 0
    w[2, 0:128].view(np.uint16)[:8] = np.arange(1, 9)  # fp16 subnormals -> scale floor
    w[2, 128:256] = (np.arange(128) - 64).astype(np.float16) * np.float16(2.0 ** -20)  # subnormal spread
    w[3, 0:128] = np.float16(1e-3) * (np.arange(128) % 7).astype(np.float16)
    w[3, 128:256] = -np.abs(w[3, 128:256])           # all-negative group
    w[4, 0:128] = np.float16(60000.0) * np.sign(w[4, 0:128])  # huge range
    return w


@pytest.mark.parametrize("bits", BITS)
def test_quantize_bit_exact_with_edge_groups(bits):
    w = edge_matrix(48, 1280, 100 + bits)
    ref = oracle.quantize(w, bits)
    got = GpuWeight(w, bits).host()
    for key in ("codes", "scales", "zeros"):
        assert np.array_equal(got[key], ref[key]), key
    assert not got["rowptr"].any()


@pytest.mark.parametrize("bits", (3, 4))
def test_quantize_outliers_bit_exact(bits):
    n, k, frac = 64, 1024, 0.002
    w = workloads.weights_fp16(n, k, 200 + bits)
    workloads.plant_outliers(w, frac, 200 + bits)
    # a run of equal magnitudes straddling the threshold: ties go to the lower index
    w[5, 10:20] = np.float16(2.5)
    w[9, 0:5] = np.float16(-2.5)
    ref = oracle.quantize(w, bits, frac)
    g = GpuWeight(w, bits, frac)
    assert g.nnz == len(ref["col"])
    got = g.host()
    for key in ("codes", "scales", "zeros", "rowptr", "col", "val"):
        assert np.array_equal(got[key], ref[key]), key


def test_quantize_outlier_ties_exact():
    n, k = 32, 512
    w = np.zeros((n, k), np.float16)
    rng = np.random.default_rng(3)
    cand = np.sort(rng.choice(n * k, 300, replace=False))
    w.reshape(-1)[cand] = np.where(rng.integers(0, 2, 300) == 1, 1.0, -1.0).astype(np.float16)
    frac = 123.5 / (n * k)
    ref = oracle.quantize(w, 2, frac)
    got = GpuWeight(w, 2, frac).host()
    for key in ("codes", "scales", "zeros", "rowptr", "col", "val"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("layout", (0, 1))
def test_pack_unpack_bit_exact(bits, layout):
    torch, q = gpu()
    n, k = 48, 1536
    codes = np.random.default_rng(bits * 10 + layout).integers(0, 1 << bits, (n, k)).astype(np.uint8)
    want = oracle.pack_device(codes, bits) if layout == 1 else oracle.pack_canonical(codes, bits)
    d = q.desc(bits, n, k, layout)
    c = torch.from_numpy(codes).cuda()
    p = torch.empty(q.qp_packed_bytes(d), dtype=torch.uint8, device="cuda")
    q.qpack_pack(d, c, p)
    assert np.array_equal(p.cpu().numpy(), want)
    back = torch.empty_like(c)
    q.qpack_unpack(d, p, back)
    assert np.array_equal(back.cpu().numpy(), codes)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_quantize_layer_4096_full(bits):
    """The 4096x4096 layer of the single-layer sweep at full size, bit-exact."""
    w = workloads.layer_weights(1 if bits == 4 else 2)
    ref = oracle.quantize(w, bits)
    g = GpuWeight(w, bits)
    got = g.host()
    for key in ("codes", "scales", "zeros"):
        assert np.array_equal(got[key], ref[key]), key
    # the device-layout bytes too
    assert np.array_equal(g.packed.cpu().numpy(), oracle.pack_device(ref["codes"], bits))


@pytest.mark.timeout(600)
def test_quantize_prefill_full_with_outliers():
    """28672 x 8192 with 234,881 planted outliers: the held-out set is exactly the planted
    set, and the dense part is bit-exact with the oracle's group quantizer."""
    w, pos = workloads.prefill_weights()
    g = GpuWeight(w, 4, workloads.PREFILL_OUTLIER_FRAC)
    got = g.host()
    assert g.nnz == len(pos) == 234_881
    rows = np.repeat(np.arange(w.shape[0]), np.diff(got["rowptr"]))
    flat = rows.astype(np.int64) * w.shape[1] + got["col"]
    assert np.array_equal(flat, pos)
    assert np.array_equal(got["val"], w.reshape(-1)[pos].view(np.uint16))
    w0 = w.copy()
    w0.reshape(-1)[pos] = 0
    for r0 in (0, 9000, 28000):  # three row bands through the oracle (fast, no sort)
        ref = oracle.quantize(w0[r0:r0 + 640], 4)
        for key in ("codes", "scales", "zeros"):
            assert np.array_equal(got[key][r0:r0 + 640], ref[key]), (key, r0)
