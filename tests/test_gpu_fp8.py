"""GPU parity of fp8 block scales with an fp16 fallback (mixed-bit page, s2.3: 8-bit float scales
take 2-bit groups of 32 to 2.25 bits per weight; the few blocks below the fp8 range keep fp16
scales): the quantizer bit for bit against the oracle (codes, scale bytes, zero points, row
factors, fallback lists and counts), and the decode GEMV reading those scales against the
oracle's fp64 product of the same weights within parity.TOL."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu


class GpuWeightFp8:
    """fp8-scale weight quantized and packed on the device through the C ABI."""

    def __init__(self, w_fp16: np.ndarray, bits: int, g: int, sym: bool, fb_stride: int = 8, layout: int = 1):
        torch, q = gpu()
        n, k = w_fp16.shape
        dev = torch.device("cuda")
        self.n, self.k, self.g, self.sym, self.fb_stride = n, k, g, sym, fb_stride
        mode = q.QP_ZERO_MIDPOINT if sym else q.QP_ZERO_STORED
        self.desc = q.desc(bits, n, k, layout, group_size=g, zero_mode=mode, scale_format=q.QP_SCALE_FP8)
        G = k // g
        w = torch.from_numpy(np.ascontiguousarray(w_fp16).view(np.int16)).to(dev)
        self.codes = torch.empty((n, k), dtype=torch.uint8, device=dev)
        self.sc8 = torch.full((n, G), 0xEE, dtype=torch.uint8, device=dev)
        self.zeros = None if sym else torch.full((n, G), 0xEE, dtype=torch.uint8, device=dev)
        self.factors = torch.empty(n, dtype=torch.float32, device=dev)
        self.fb = torch.zeros((n, max(fb_stride, 1)), dtype=torch.int16, device=dev)
        self.counts = torch.full((n,), -1, dtype=torch.int32, device=dev)
        q.qpack_quantize_fp8(self.desc, w, k, self.codes, self.sc8, self.zeros, self.factors,
                             self.fb if fb_stride else None, fb_stride, self.counts)
        self.packed = torch.empty(q.qp_packed_bytes(self.desc), dtype=torch.uint8, device=dev)
        q.qpack_pack(self.desc, self.codes, self.packed)

    def handle(self):
        _, q = gpu()
        return q.weight_fp8(self.packed, self.sc8, self.factors, self.fb if self.fb_stride else None,
                            self.fb_stride, self.zeros)

    def host(self) -> dict:
        return dict(codes=self.codes.cpu().numpy(), sc8=self.sc8.cpu().numpy(),
                    zeros=None if self.sym else self.zeros.cpu().numpy(), factors=self.factors.cpu().numpy(),
                    fb=self.fb.cpu().numpy().view(np.uint16)[:, : self.fb_stride], counts=self.counts.cpu().numpy())


def gemv(gw: GpuWeightFp8, x: np.ndarray) -> np.ndarray:
    torch, q = gpu()
    m, k = x.shape
    y = torch.empty((m, gw.n), dtype=torch.int16, device="cuda")
    q.qlinear_gemv(gw.desc, gw.handle(), to_dev_fp16(x), k, m, y, gw.n)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


def plant_fallbacks(w: np.ndarray, g: int, seed: int, rows=(0, 5, 9, 17, 30), per_row=3):
    """Rows whose first group is scaled up 20000x and `per_row` other groups down 2x: their
    scales sit ~40000x below the row's largest, beyond E4M3's 2^14 range below 256, so they
    fall back; the rest are scaled up 100x and stay inside the fp8 range."""
    rng = np.random.default_rng(seed)
    G = w.shape[1] // g
    for r in rows:
        keep = set(rng.choice(np.arange(1, G), per_row, replace=False).tolist())
        for c in range(G):
            f = 20000.0 if c == 0 else (0.5 if c in keep else 100.0)
            w[r, c * g:(c + 1) * g] = (w[r, c * g:(c + 1) * g].astype(np.float32) * f).astype(np.float16)


@pytest.mark.parametrize("g", (32, 64, 128))
@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("sym", (False, True))
def test_quantize_fp8_bit_exact(g, bits, sym):
    """Every output of the fp8 quantizer equals the oracle's: planted fallback groups, an
    all-zero group and an all-zero row, and a row with more fallbacks (12) than slots (8)."""
    print(f"quantize fp8 g={g} bits={bits} sym={sym}", flush=True)
    w = workloads.weights_fp16(48, 2048, 2000 + bits + g)
    plant_fallbacks(w, g, 2000 + bits)
    w[3, 128:256] = 0
    w[11] = 0
    plant_fallbacks(w, g, 2100 + bits, rows=(21,), per_row=12)
    want = oracle.quantize_fp8(w, bits, g, sym=sym, fb_stride=8)
    got = GpuWeightFp8(w, bits, g, sym).host()
    assert want["counts"][21] == 12 and want["counts"][0] == 3
    for key in ("codes", "sc8", "factors", "fb", "counts"):
        assert np.array_equal(got[key], want[key]), key
    if not sym:
        assert np.array_equal(got["zeros"], want["zeros"])


def test_quantize_fp8_layer_4096_two_bit_groups_of_32():
    """The 4096 x 4096 layer at the page's 2.25-bit setting: 2-bit symmetric groups of 32."""
    w = workloads.layer_weights(2)
    want = oracle.quantize_fp8(w, 2, 32, sym=True)
    got = GpuWeightFp8(w, 2, 32, True).host()
    for key in ("codes", "sc8", "factors", "counts"):
        assert np.array_equal(got[key], want[key]), key


@pytest.mark.parametrize("g", (32, 64, 128))
@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("m", (1, 3, 16))
def test_gemv_fp8(g, bits, m):
    """6 k-tiles over 8 waves, fallback groups in five rows, affine and symmetric groups."""
    n, k = 48, 1536
    for sym in (False, True):
        print(f"gemv fp8 g={g} bits={bits} m={m} sym={sym}", flush=True)
        w = workloads.weights_fp16(n, k, 2200 + bits + g)
        plant_fallbacks(w, g, 2200 + bits)
        x = workloads.activations_fp16(m, k, 2200 + bits)
        r = oracle.linear_fp8(x, oracle.quantize_fp8(w, bits, g, sym=sym))
        y = gemv(GpuWeightFp8(w, bits, g, sym), x)
        assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("g", (32, 64, 128))
@pytest.mark.parametrize("bits", (2, 4, 6))
def test_gemv_fp8_fallback_groups_alone(g, bits):
    """Rows whose output comes from fallback groups only: the first group of the even rows is
    large (it sets the row factor) and every other group of those rows falls back; x is zero
    over the first group, so y of an even row is the fallback groups' sum alone, through the
    fp16 scales of the fallback list.  Odd rows stay ordinary fp8 rows in the same tiles."""
    n, k, m = 32, 1024, 5
    print(f"gemv fp8 fallback-only g={g} bits={bits}", flush=True)
    w = workloads.weights_fp16(n, k, 2300 + bits, std=0.002)
    w[0::2, :g] = workloads.weights_fp16(n // 2, g, 2301, std=100.0)
    x = workloads.activations_fp16(m, k, 2300 + bits)
    x[:, :g] = 0
    G = k // g
    qd = oracle.quantize_fp8(w, bits, g, sym=False, fb_stride=G)
    assert (qd["counts"][0::2] == G - 1).all() and (qd["counts"][1::2] == 0).all()
    r = oracle.linear_fp8(x, qd)
    y = gemv(GpuWeightFp8(w, bits, g, False, fb_stride=G), x)
    assert rel_err(y, r) <= TOL, report(y, r)
    assert rel_err(y[:, 0::2], r[:, 0::2]) <= TOL, report(y[:, 0::2], r[:, 0::2])


@pytest.mark.parametrize("m", (1, 8))
def test_gemv_fp8_wide_matrix_four_wave_kernel(m):
    """n = 8192 (512 row blocks): the 4-wave GEMV geometry."""
    n, k = 8192, 512
    w = workloads.weights_fp16(n, k, 2400)
    plant_fallbacks(w, 32, 2400, rows=(1, 4000, 8191))
    x = workloads.activations_fp16(m, k, 2400)
    r = oracle.linear_fp8(x, oracle.quantize_fp8(w, 2, 32, sym=True))
    y = gemv(GpuWeightFp8(w, 2, 32, True), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("m", (1, 16))
def test_gemv_fp8_layer_4096(m):
    """The 4096 x 4096 layer at 2-bit symmetric groups of 32 with fp8 scales, all outputs."""
    w = workloads.layer_weights(2)
    x = workloads.activations_fp16(m, 4096, workloads.seed_for(2))
    r = oracle.linear_fp8(x, oracle.quantize_fp8(w, 2, 32, sym=True))
    y = gemv(GpuWeightFp8(w, 2, 32, True), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("m", (1, 2, 9, 16))
def test_gemv_fp8_single_tile_and_block(m):
    """The smallest shapes: one 16-row block and one 256-k tile (k = 256), every group size,
    fallbacks in the last group of a row."""
    for g in (32, 64, 128):
        w = workloads.weights_fp16(16, 256, 2500 + g)
        w[3, :g] *= np.float16(400.0)
        w[3, 256 - g:] = (w[3, 256 - g:].astype(np.float32) * 0.01).astype(np.float16)
        x = workloads.activations_fp16(m, 256, 2500 + g)
        qd = oracle.quantize_fp8(w, 4, g, sym=False)
        assert qd["counts"][3] >= 1 and qd["sc8"][3, -1] >= 0x80
        y = gemv(GpuWeightFp8(w, 4, g, False), x)
        r = oracle.linear_fp8(x, qd)
        assert rel_err(y, r) <= TOL, report(y, r)


def test_gemv_fp8_without_fallback_list():
    """fb_stride = 0 (no list passed): weights without fallbacks run unchanged."""
    w = workloads.weights_fp16(64, 1024, 2600)
    x = workloads.activations_fp16(4, 1024, 2600)
    qd = oracle.quantize_fp8(w, 3, 64, sym=True, fb_stride=0)
    assert qd["counts"].sum() == 0
    y = gemv(GpuWeightFp8(w, 3, 64, True, fb_stride=0), x)
    r = oracle.linear_fp8(x, qd)
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemv_fp8_fallback_index_past_the_list_reads_the_last_slot():
    """A row with more fallbacks than slots: bytes 0x80 | j with j >= fb_stride are malformed;
    the GEMV reads the row's last slot for them, so the output equals the oracle's product with
    those groups' scales replaced by that slot's (and stays inside the buffers)."""
    g, n, k, m = 32, 16, 512, 3
    w = workloads.weights_fp16(n, k, 2700, std=0.002)
    w[5, :g] = workloads.weights_fp16(1, g, 2701, std=100.0)  # row 5: 15 fallbacks, 4 slots
    x = workloads.activations_fp16(m, k, 2700)
    x[:, :g] = 0
    qd = oracle.quantize_fp8(w, 4, g, sym=False, fb_stride=4)
    assert qd["counts"][5] == k // g - 1
    fb_last = np.float32(oracle.half_value(int(qd["fb"][5, 3])))
    sc = qd["scales_f32"].copy()
    for gi in range(k // g):
        b = int(qd["sc8"][5, gi])
        if b & 0x80 and (b & 0x7F) >= 4:
            sc[5, gi] = fb_last
    r = oracle.linear_fp8(x, dict(qd, scales_f32=sc))
    y = gemv(GpuWeightFp8(w, 4, g, False, fb_stride=4), x)
    assert rel_err(y, r) <= TOL, report(y, r)


def gemm(gw: GpuWeightFp8, x: np.ndarray) -> np.ndarray:
    torch, q = gpu()
    m, k = x.shape
    y = torch.empty((m, gw.n), dtype=torch.int16, device="cuda")
    q.qlinear_gemm(gw.desc, gw.handle(), to_dev_fp16(x), k, m, y, gw.n, None, 0)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


@pytest.mark.parametrize("g", (32, 64, 128))
@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
@pytest.mark.parametrize("m", (17, 130))
def test_gemm_fp8(g, bits, m):
    """The prefill GEMM on fp8 scales: a partial last weight tile (n = 560), a ragged activation
    block (m = 17) or a full one plus a ragged one (m = 130), fallback groups in five rows,
    affine and symmetric groups."""
    n, k = 560, 1536
    for sym in (False, True):
        print(f"gemm fp8 g={g} bits={bits} m={m} sym={sym}", flush=True)
        w = workloads.weights_fp16(n, k, 2800 + bits + g)
        plant_fallbacks(w, g, 2800 + bits, rows=(0, 5, 300, 513, 559))
        x = workloads.activations_fp16(m, k, 2800 + bits)
        qd = oracle.quantize_fp8(w, bits, g, sym=sym)
        assert qd["counts"][300] == 3
        y = gemm(GpuWeightFp8(w, bits, g, sym), x)
        r = oracle.linear_fp8(x, qd)
        assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("g", (32, 128))
def test_gemm_fp8_fallback_groups_alone(g):
    """Even rows whose outputs come from fallback groups only (x zero over their one large
    group), through the GEMM's fallback path."""
    n, k, m = 256, 1024, 64
    w = workloads.weights_fp16(n, k, 2900 + g, std=0.002)
    w[0::2, :g] = workloads.weights_fp16(n // 2, g, 2901, std=100.0)
    x = workloads.activations_fp16(m, k, 2900 + g)
    x[:, :g] = 0
    G = k // g
    qd = oracle.quantize_fp8(w, 4, g, sym=False, fb_stride=G)
    assert (qd["counts"][0::2] == G - 1).all()
    y = gemm(GpuWeightFp8(w, 4, g, False, fb_stride=G), x)
    r = oracle.linear_fp8(x, qd)
    assert rel_err(y[:, 0::2], r[:, 0::2]) <= TOL, report(y[:, 0::2], r[:, 0::2])
    assert rel_err(y, r) <= TOL, report(y, r)


def test_gemm_fp8_layer_4096_prefill():
    """The 4096 x 4096 layer at the page's 2.25-bit setting (2-bit symmetric groups of 32, fp8
    scales), M = 512: every output against the oracle."""
    w = workloads.layer_weights(2)
    x = workloads.activations_fp16(512, 4096, workloads.seed_for(2))
    qd = oracle.quantize_fp8(w, 2, 32, sym=True)
    y = gemm(GpuWeightFp8(w, 2, 32, True), x)
    r = oracle.linear_fp8(x, qd)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("g", (32, 128))
@pytest.mark.parametrize("m", (1, 5))
def test_gemv_batch_fp8(g, m):
    """Independent fp8-scale problems of 2, 4 and 6 bits (and widths, fallback groups planted)
    in one qlinear_gemv_batch launch: each output against the oracle's product."""
    torch, q = gpu()
    k = 1024
    shapes = ((2, 192), (4, 64), (6, 320), (2, 16))
    ws, ys, refs = [], [], []
    x = workloads.activations_fp16(m, k, 3200 + g)
    xd = to_dev_fp16(x)
    for i, (bits, n) in enumerate(shapes):
        w = workloads.weights_fp16(n, k, 3200 + 7 * i + bits)
        plant_fallbacks(w, g, 3300 + i, rows=(0, n - 1), per_row=2)
        qd = oracle.quantize_fp8(w, bits, g, sym=(i % 2 == 1))
        ws.append(GpuWeightFp8(w, bits, g, i % 2 == 1))
        ys.append(torch.empty((m, n), dtype=torch.int16, device="cuda"))
        refs.append(oracle.linear_fp8(x, qd))
    q.qlinear_gemv_batch([q.gemv_problem(gw.desc, gw.handle(), xd, k, m, y, gw.n) for gw, y in zip(ws, ys)])
    torch.cuda.synchronize()
    for (bits, n), y, r in zip(shapes, ys, refs):
        yh = from_dev_fp16(y)
        assert rel_err(yh, r) <= TOL, (bits, n, report(yh, r))
