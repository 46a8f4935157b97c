"""GPU parity of the matrix-core GEMMs for the metadata variants of the mixed-bit page (s2.3):
groups of 32 and 64, symmetric groups, and zero points stored in b bits, in the prefill GEMM
(with and without outliers, full and ragged activation tiles), the grouped expert GEMM, the
routed-expert FFN and the int8-activation GEMM.  Each result is checked against the oracle's
fp64 product within parity.TOL; launches reading b-bit zero points are also checked element
for element against the same launch reading the same zero points as bytes (identical values,
identical arithmetic)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16
from test_gpu_moe import Experts, check_ffn, dev, expected_dispatch, flip_bound, run_ffn, small_routing

pytestmark = pytest.mark.gpu
BITS = (2, 3, 4, 5, 6)


def gemm(g: GpuWeight, x: np.ndarray, with_csr=True, byte_zeros=False):
    torch, q = gpu()
    m, k = x.shape
    y = torch.empty((m, g.n), dtype=torch.int16, device="cuda")
    nnz = g.nnz if with_csr else 0
    wsb = q.qlinear_gemm_workspace_bytes(g.desc, m, nnz)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    d, h = g.desc, g.handle(with_csr)
    if byte_zeros:  # the same weight with its zero points as bytes
        d = q.desc(g.bits, g.n, g.k, group_size=g.g)
        h = q.weight(g.packed, g.scales, g.zeros_u8, h.csr_rowptr, h.csr_col, h.csr_val, h.nnz)
    q.qlinear_gemm(d, h, to_dev_fp16(x), k, m, y, g.n, ws, wsb)
    torch.cuda.synchronize()
    return from_dev_fp16(y)


@pytest.mark.parametrize("gs", (32, 64))
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", (17, 130))
def test_gemm_small_groups_with_outliers(gs, bits, m):
    """A partial last weight tile (n = 560), a ragged activation block (m = 17) or a full one
    plus a ragged one (m = 130), outliers added back."""
    print(f"gemm g={gs} bits={bits} m={m}", flush=True)
    n, k, frac = 560, 1536, 0.002
    w = workloads.weights_fp16(n, k, 1000 + bits + gs)
    workloads.plant_outliers(w, frac, 1000 + bits)
    x = workloads.activations_fp16(m, k, 1000 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, frac, g=gs))
    y = gemm(GpuWeight(w, bits, frac, g=gs), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.parametrize("gs", (32, 64, 128))
@pytest.mark.parametrize("bits", BITS)
def test_gemm_packed_zeros(gs, bits):
    """b-bit zero points (row streams of 1536 / g fields, ending inside a word at most widths)."""
    print(f"gemm packed zeros g={gs} bits={bits}", flush=True)
    n, k, m = 288, 1536, 150
    w = workloads.weights_fp16(n, k, 1100 + bits + gs)
    x = workloads.activations_fp16(m, k, 1100 + bits)
    g = GpuWeight(w, bits, g=gs, packed_zeros=True)
    y = gemm(g, x)
    r = oracle.linear(x, oracle.quantize(w, bits, g=gs))
    assert rel_err(y, r) <= TOL, report(y, r)
    assert np.array_equal(y, gemm(g, x, byte_zeros=True))


@pytest.mark.parametrize("gs", (32, 64))
@pytest.mark.parametrize("bits", (2, 3))
def test_gemm_symmetric_small_groups(gs, bits):
    """The page's pairing: symmetric groups of 32 / 64 at 2 and 3 bits."""
    n, k, m = 256, 2048, 128
    w = workloads.weights_fp16(n, k, 1200 + bits + gs)
    x = workloads.activations_fp16(m, k, 1200 + bits)
    r = oracle.linear(x, oracle.quantize(w, bits, g=gs, sym=True))
    y = gemm(GpuWeight(w, bits, sym=True, g=gs), x)
    assert rel_err(y, r) <= TOL, report(y, r)


@pytest.mark.timeout(600)
def test_gemm_layer_4096_groups_of_32_prefill():
    """The 4096 x 4096 layer at 2 bits, g = 32, packed zero points, M = 512 (four full
    activation blocks): 256 sampled weight rows x all 512 rows recomputed by the oracle."""
    w = workloads.layer_weights(2)
    x = workloads.activations_fp16(512, 4096, workloads.seed_for(2))
    g = GpuWeight(w, 2, g=32, packed_zeros=True)
    y = gemm(g, x)
    ns = np.sort(np.random.default_rng(32).choice(4096, 256, replace=False))
    r = oracle.linear(x, oracle.quantize(w[ns], 2, g=32))
    assert rel_err(y[:, ns], r) <= TOL, report(y[:, ns], r)


@pytest.mark.parametrize("gs,packed", ((32, False), (64, True), (32, True)))
@pytest.mark.parametrize("epilogue", ("rows_f32", "none", "swiglu"))
def test_grouped_small_groups(gs, packed, epilogue):
    """Routed expert rows on both workgroup geometries (23 and 225 rows per expert on
    average), with small groups and b-bit zero points, through each epilogue."""
    torch, q = gpu()
    print(f"grouped g={gs} packed={packed} {epilogue}", flush=True)
    for sizes in ([30, 33, 0, 1, 40, 16, 17, 50], [300, 0, 290, 311]):
        E, D, F = len(sizes), 512, 256
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        R = int(offsets[-1])
        x = workloads.activations_fp16(R, D, 1300 + gs)
        raw = [(workloads.weights_fp16(F, D, 1310 + e), workloads.weights_fp16(F, D, 1330 + e)) for e in range(E)]
        gu_raw = [workloads.interleave_row_blocks(a, b) for a, b in raw]
        ws = [GpuWeight(m, 4, g=gs, packed_zeros=packed) for m in gu_raw]
        hs = [w.handle() for w in ws]
        if epilogue == "rows_f32":
            y = torch.empty((R, 2 * F), dtype=torch.float32, device="cuda")
            q.qlinear_grouped_gemm(ws[0].desc, hs, to_dev_fp16(x), D, None, dev(offsets), R, q.QP_EPI_ROWS_F32, y,
                                   2 * F)
        elif epilogue == "none":
            y = torch.empty((R, 2 * F), dtype=torch.int16, device="cuda")
            q.qlinear_grouped_gemm(ws[0].desc, hs, to_dev_fp16(x), D, None, dev(offsets), R, q.QP_EPI_NONE, y, 2 * F)
        else:
            y = torch.empty((R, F), dtype=torch.int16, device="cuda")
            q.qlinear_grouped_gemm(ws[0].desc, hs, to_dev_fp16(x), D, None, dev(offsets), R, q.QP_EPI_SWIGLU, y, F)
        torch.cuda.synchronize()
        y = y.cpu().numpy() if epilogue == "rows_f32" else from_dev_fp16(y)
        for e in range(E):
            rows = np.arange(offsets[e], offsets[e + 1])
            if not len(rows):
                continue
            if epilogue == "swiglu":
                gq, uq = oracle.quantize(raw[e][0], 4, g=gs), oracle.quantize(raw[e][1], 4, g=gs)
                for row in rows[:: max(1, len(rows) // 8)]:
                    v = oracle.swiglu_act(x[row], gq, uq)
                    # one fp16 rounding of silu(g) * u: within an ulp of the fp64 value, floored
                    ulp = np.spacing(np.abs(v).astype(np.float16)).astype(np.float64)
                    err = np.abs(y[row].astype(np.float64) - v)
                    assert (err <= ulp + TOL * np.sqrt(np.mean(v * v))).all(), (e, row, err.max())
            else:
                r = oracle.linear(x[rows], oracle.quantize(gu_raw[e], 4, g=gs))
                assert rel_err(y[rows], r) <= TOL, (e, report(y[rows], r))


@pytest.mark.parametrize("gs,packed", ((64, False), (32, True)))
@pytest.mark.parametrize("F", (768, 1024), ids=("down-one-pass", "down-two-k-halves"))
def test_moe_ffn_small_groups(gs, packed, F):
    """The whole expert FFN with small groups (and b-bit zero points): the down projection in
    one pass, or in two k halves whose zero-point fields start mid-row."""
    print(f"moe ffn g={gs} packed={packed} F={F}", flush=True)
    E, D, T = 5, 512, 37
    ex = Experts(E, D, F, 3, stream=80 + gs, g=gs, packed_zeros=packed)
    x = workloads.activations_fp16(T, D, 81)
    ids, wts = small_routing(T, E, 82)
    y = run_ffn(ex, x, ids, wts)
    r = oracle.moe_ffn(x, ids, wts, *ex.oracle_sets(set(range(E))))
    check_ffn(y, r, flip_bound(ex, x, ids, wts))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6))
def test_gemm_a8_packed_zeros(bits):
    """The int8-activation GEMM reading b-bit zero points equals the same launch reading them
    as bytes, element for element, and the oracle within TOL."""
    torch, q = gpu()
    n, k, m = 288, 1536, 100
    w = workloads.weights_fp16(n, k, 1400 + bits)
    x = workloads.activations_fp16(m, k, 1400 + bits)
    g = GpuWeight(w, bits, packed_zeros=True)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sx = torch.empty(m, dtype=torch.float32, device="cuda")
    q.qact_quantize(to_dev_fp16(x), k, m, k, xq, sx)
    ys = []
    for d, h in ((g.desc, g.handle(False)), (q.desc(bits, n, k), q.weight(g.packed, g.scales, g.zeros_u8))):
        y = torch.empty((m, n), dtype=torch.int16, device="cuda")
        q.qlinear_gemm_a8(d, h, xq, sx, m, y, n)
        torch.cuda.synchronize()
        ys.append(from_dev_fp16(y))
    assert np.array_equal(ys[0], ys[1])
    rq, rs = oracle.act_quantize(x)
    r = oracle.linear_a8(rq, rs, oracle.quantize(w, bits))
    assert rel_err(ys[0], r) <= TOL, report(ys[0], r)
