"""GPU parity for zero points stored in b bits (QP_ZERO_PACKED; mixed-bit page, s2.3).

qpack_pack_zeros against the oracle's packer, bit for bit; the GEMV and the batched GEMV
reading packed zero points against the oracle's fp64 product within parity.TOL, and against
the same launch reading byte zero points, element for element (the zero point values, and so
the arithmetic, are identical)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu


class PackedZeroWeight:
    """An affine weight quantized and packed through the C ABI, with its zero points both as
    bytes (qpack_quantize's output) and packed in b bits (qpack_pack_zeros)."""

    def __init__(self, w_fp16: np.ndarray, bits: int, g: int):
        torch, q = gpu()
        n, k = w_fp16.shape
        self.n, self.k, self.bits, self.g = n, k, bits, g
        self.dp = q.desc(bits, n, k, group_size=g, zero_mode=q.QP_ZERO_PACKED)
        self.ds = q.desc(bits, n, k, group_size=g)
        w = to_dev_fp16(w_fp16)
        self.codes = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((n, k // g), dtype=torch.int16, device="cuda")
        self.zeros = torch.empty((n, k // g), dtype=torch.uint8, device="cuda")
        q.qpack_quantize(self.dp, w, k, 0.0, self.codes, self.scales, self.zeros)
        self.packed = torch.empty(q.qp_packed_bytes(self.dp), dtype=torch.uint8, device="cuda")
        q.qpack_pack(self.dp, self.codes, self.packed)
        self.pz = torch.full((q.qp_zero_bytes(self.dp),), 0xA5, dtype=torch.uint8, device="cuda")
        q.qpack_pack_zeros(self.dp, self.zeros, self.pz)
        torch.cuda.synchronize()

    def packed_handle(self):
        _, q = gpu()
        return q.weight(self.packed, self.scales, self.pz)

    def byte_handle(self):
        _, q = gpu()
        return q.weight(self.packed, self.scales, self.zeros)


def gemv(d, h, x, n):
    torch, q = gpu()
    m, k = x.shape
    xd = to_dev_fp16(x)
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    q.qlinear_gemv(d, h, xd, k, m, y, n)
    torch.cuda.synchronize()
    return from_dev_fp16(y).astype(np.float64)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("g", (32, 64, 128))
def test_pack_zeros_bit_exact(bits, g):
    print(f"pack zeros bits={bits} g={g}", flush=True)
    w = workloads.weights_fp16(48, 1280, 940 + bits + g)
    pw = PackedZeroWeight(w, bits, g)
    ref = oracle.quantize(w, bits, g=g)
    assert np.array_equal(pw.zeros.cpu().numpy(), ref["zeros"])
    want = oracle.pack_zeros(ref["zeros"], bits).reshape(-1)
    assert np.array_equal(pw.pz.cpu().numpy(), want)


@pytest.mark.parametrize("bits", (2, 3, 5, 6))
@pytest.mark.parametrize("g", (32, 64, 128))
@pytest.mark.parametrize("m", (1, 8, 16))
def test_gemv_packed_zeros(bits, g, m):
    print(f"gemv packed zeros bits={bits} g={g} m={m}", flush=True)
    n, k = 64, 1280  # 1280 / g groups per row: row streams that end inside a 32-bit word
    w = workloads.weights_fp16(n, k, 950 + bits + g)
    x = workloads.activations_fp16(m, k, 950 + bits)
    pw = PackedZeroWeight(w, bits, g)
    y = gemv(pw.dp, pw.packed_handle(), x, n)
    r = oracle.linear(x, oracle.quantize(w, bits, g=g))
    assert rel_err(y, r) <= TOL, report(y, r)
    assert np.array_equal(y, gemv(pw.ds, pw.byte_handle(), x, n))


@pytest.mark.parametrize("g", (32, 128))
def test_gemv_packed_zeros_wide_layer(g):
    """A 4096-wide layer (k/g groups per row fill whole words) at 2 and 5 bits."""
    for bits in (2, 5):
        w = workloads.layer_weights(2)
        x = workloads.activations_fp16(1, 4096, workloads.seed_for(2))
        pw = PackedZeroWeight(w, bits, g)
        y = gemv(pw.dp, pw.packed_handle(), x, 4096)
        r = oracle.linear(x, oracle.quantize(w, bits, g=g))
        assert rel_err(y, r) <= TOL, (bits, report(y, r))


@pytest.mark.parametrize("g", (32, 64, 128))
def test_gemv_batch_packed_zeros(g):
    """Mixed bit widths in one launch, all with packed zero points, against single launches."""
    torch, q = gpu()
    k = 1280
    x = workloads.activations_fp16(4, k, 960)
    xd = to_dev_fp16(x)
    ws, probs, outs, refs = [], [], [], []
    for i, bits in enumerate((2, 3, 5, 6)):
        n = 32 * (i + 1)
        pw = PackedZeroWeight(workloads.weights_fp16(n, k, 961 + i), bits, g)
        y = torch.empty((4, n), dtype=torch.int16, device="cuda")
        ws.append(pw)
        outs.append(y)
        probs.append(q.gemv_problem(pw.dp, pw.packed_handle(), xd, k, 4, y, n))
        refs.append(gemv(pw.dp, pw.packed_handle(), x, n))
    q.qlinear_gemv_batch(probs)
    torch.cuda.synchronize()
    for y, r in zip(outs, refs):
        assert np.array_equal(from_dev_fp16(y).astype(np.float64), r)
