"""GPU parity of the routed-expert path on fp8-scale weights (mixed-bit page, s2.3: E4M3 group
scales with a per-row factor and an fp16 fallback list; MoE page, s4.2: the expert FFN): each
grouped projection (fp32 rows, fp16 rows, the SwiGLU epilogue) and the whole FFN (qmoe_ffn)
against the oracle's fp64 products over the same weights.  Fallback groups planted in gate and
down rows of every expert exercise the fallback list.  The FFN check allows the near-tie fp16
flips of its intermediate, as for fp16 scales."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, from_dev_fp16, gpu, rel_err, report, to_dev_fp16
from test_gpu_fp8 import GpuWeightFp8
from test_gpu_moe import check_ffn, dev, expected_dispatch, near_tie, small_routing

pytestmark = pytest.mark.gpu

CASES = ((2, 32, True), (4, 128, False), (3, 64, True), (5, 32, False), (6, 128, True))


def shrink_groups(w: np.ndarray, g: int, row: int, groups):
    """Scale the given groups of one row by 2^-16: their scales fall more than E4M3's 2^-14
    below the row's largest, so they take fp16 fallback scales; magnitudes elsewhere stay."""
    for c in groups:
        w[row, c * g:(c + 1) * g] = (w[row, c * g:(c + 1) * g].astype(np.float32) * 2.0 ** -16).astype(np.float16)


class ExpertsFp8:
    """Gate/up interleaved by 16-row blocks, and down, quantized with fp8 scales on the GPU; the
    oracle's quantization of the same matrices beside them."""

    def __init__(self, E, D, F, bits, g, sym, stream):
        self.D, self.F = D, F
        self.gate_up, self.down, self.qd, self.raw = [], [], [], []
        for e in range(E):
            gt, u, d = workloads.moe_expert(e, D, F, stream)
            shrink_groups(gt, g, 0, (1, 3))
            shrink_groups(gt, g, 17, (0, 2))
            shrink_groups(d, g, 3, (2, 5))
            self.raw.append((gt, u, d))
            self.gate_up.append(GpuWeightFp8(workloads.interleave_row_blocks(gt, u), bits, g, sym))
            self.down.append(GpuWeightFp8(d, bits, g, sym))
            self.qd.append(tuple(oracle.quantize_fp8(m, bits, g, sym=sym) for m in (gt, u, d)))
        assert self.qd[0][0]["counts"][0] == 2 and self.qd[0][2]["counts"][3] == 2

    def handles(self, which):
        return [w.handle() for w in (self.gate_up if which == "gu" else self.down)]


@pytest.mark.parametrize("bits,g,sym", CASES)
def test_grouped_fp8_projections(bits, g, sym):
    """gate/up as fp32 and fp16 rows and through the SwiGLU epilogue on gathered token rows,
    and down on the oracle's fp16 intermediate, expert by expert (one expert gets no rows)."""
    torch, q = gpu()
    print(f"grouped fp8 bits={bits} g={g} sym={sym}", flush=True)
    E, D, F, T = 5, 512, 768, 37
    ex = ExpertsFp8(E, D, F, bits, g, sym, 3000 + bits)
    x = workloads.activations_fp16(T, D, 3001)
    ids, wts = small_routing(T, E, 3002)
    order, offsets, row_src, _ = expected_dispatch(ids, E)
    R = len(order)
    xd, off_d, src_d = to_dev_fp16(x), dev(offsets), dev(row_src)
    gud = ex.gate_up[0].desc
    y32 = torch.empty((R, 2 * F), dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(gud, ex.handles("gu"), xd, D, src_d, off_d, R, q.QP_EPI_ROWS_F32, y32, 2 * F)
    y16 = torch.empty((R, 2 * F), dtype=torch.int16, device="cuda")
    q.qlinear_grouped_gemm(gud, ex.handles("gu"), xd, D, src_d, off_d, R, q.QP_EPI_NONE, y16, 2 * F)
    act = torch.empty((R, F), dtype=torch.int16, device="cuda")
    q.qlinear_grouped_gemm(gud, ex.handles("gu"), xd, D, src_d, off_d, R, q.QP_EPI_SWIGLU, act, F)
    torch.cuda.synchronize()
    y32, y16, act = y32.cpu().numpy(), from_dev_fp16(y16), from_dev_fp16(act)
    a_ref = np.zeros((R, F), np.float16)
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows) == 0:
            continue
        gq, uq, _ = ex.qd[e]
        xr = x[row_src[rows]]
        r = oracle.linear_fp8(xr, oracle.quantize_fp8(workloads.interleave_row_blocks(*ex.raw[e][:2]), bits, g, sym=sym))
        assert rel_err(y32[rows], r) <= TOL, (e, report(y32[rows], r))
        assert rel_err(y16[rows], r) <= TOL, (e, report(y16[rows], r))
        v = oracle.swiglu_act_fp8(xr, gq, uq)
        assert rel_err(act[rows], v) <= TOL, (e, report(act[rows], v))
        a_ref[rows] = v.astype(np.float16)
    yd = torch.empty((R, D), dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ex.down[0].desc, ex.handles("dn"), to_dev_fp16(a_ref), F, None, off_d, R,
                           q.QP_EPI_ROWS_F32, yd, D)
    torch.cuda.synchronize()
    yd = yd.cpu().numpy()
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows):
            r = oracle.linear_fp8(a_ref[rows], ex.qd[e][2])
            assert rel_err(yd[rows], r) <= TOL, (e, report(yd[rows], r))


def flip_bound_fp8(ex: ExpertsFp8, x, ids, wts):
    """Per-output worst-case effect of near-tie intermediate elements rounding the other way."""
    T, K = ids.shape
    bound = np.zeros((T, ex.D))
    for t in range(T):
        for j in range(K):
            gq, uq, dq = ex.qd[int(ids[t, j])]
            _, ulp, near = near_tie(oracle.swiglu_act_fp8(x[t:t + 1], gq, uq)[0])
            if near.any():
                cols = np.nonzero(near)[0]
                bound[t] += float(wts[t, j]) * (np.abs(oracle.dequant_fp8(dq)[:, cols]) * ulp[cols]).sum(axis=1)
    return bound


@pytest.mark.parametrize("bits,g,sym", CASES)
@pytest.mark.parametrize("F", (768, 1024), ids=("down-one-pass", "down-two-k-halves"))
def test_moe_ffn_fp8(bits, g, sym, F):
    """The whole FFN on fp8-scale experts: dispatch, gate/up with the SwiGLU epilogue, down (in
    one pass, or two k halves summed by the combine), combine."""
    torch, q = gpu()
    print(f"moe ffn fp8 bits={bits} g={g} sym={sym} F={F}", flush=True)
    E, D, T = 5, 512, 37
    ex = ExpertsFp8(E, D, F, bits, g, sym, 3100 + bits)
    x = workloads.activations_fp16(T, D, 3101)
    ids, wts = small_routing(T, E, 3102)
    ws_bytes = q.qmoe_ffn_workspace_bytes(T, 2, E, D, F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    q.qmoe_ffn(ex.gate_up[0].desc, ex.handles("gu"), ex.down[0].desc, ex.handles("dn"), to_dev_fp16(x), D, T,
               dev(ids), dev(wts), 2, out, D, ws, ws_bytes)
    torch.cuda.synchronize()
    y = from_dev_fp16(out)
    r = oracle.moe_ffn_fp8(x, ids, wts, *[[ex.qd[e][i] for e in range(E)] for i in range(3)])
    check_ffn(y, r, flip_bound_fp8(ex, x, ids, wts))
