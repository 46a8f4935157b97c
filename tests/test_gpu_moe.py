"""GPU parity for the routed-expert path (MoE page, s4.2): dispatch (bit-exact integer
work), each grouped projection against the oracle's fp64 linear layer at the standard
tolerance, the SwiGLU epilogue's fp16 rounding, and the whole FFN (qmoe_ffn).

The FFN stores its intermediate silu(g)*u in fp16 (the down projection's input is an fp16
activation).  The GPU forms g and u in fp32, the oracle in fp64, so an element whose exact
value lies within a rounding error of an fp16 midpoint may legitimately round to the other
neighbour.  One such flip moves every output of that token by ulp(a_f) * |W_down[:, f]| * p,
about 5e-5 of rms(out) -- more than the 2e-3 tolerance allows at its 1%-of-rms floor.  The
end-to-end check therefore adds, per output, the exact worst-case contribution of the
intermediate elements that sit within 1/256 fp16-ulp of a midpoint (about 100x the fp32
error of g and u); everywhere else it is the standard tolerance.  The SwiGLU test checks
that flips occur only at such near-ties.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu


def dev(a):
    torch, _ = gpu()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def expected_dispatch(ids, E):
    """Stable sort of the (token, choice) pairs by expert (numpy)."""
    T, K = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    offsets = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]).astype(np.int32)
    token_rows = np.empty(T * K, np.int64)
    token_rows[order] = np.arange(T * K)
    return order, offsets, (order // K).astype(np.int32), token_rows


def test_dispatch_exact():
    torch, q = gpu()
    T, E, K = 300, 12, 2
    ids, wts = workloads.zipf_routing(T, E, K, 1.1, 77)
    ids[ids == 5] = 4  # leave expert 5 empty
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % E, ids[:, 1])
    order, want_off, want_src, want_rows = expected_dispatch(ids, E)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(T * K, dtype=torch.int32, device="cuda")
    rw = torch.empty(T * K, dtype=torch.float32, device="cuda")
    tr = torch.empty(T * K, dtype=torch.int32, device="cuda")
    q.qmoe_dispatch(dev(ids), dev(wts), T, K, E, off, src, rw, tr)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(src.cpu().numpy(), want_src)
    assert np.array_equal(tr.cpu().numpy(), want_rows)
    assert np.array_equal(rw.cpu().numpy(), wts.reshape(-1)[order])


class Experts:
    """Gate/up interleaved by 16-row blocks, and down, quantized and packed on the GPU."""

    def __init__(self, E, D, F, bits, stream, g: int = 128, packed_zeros: bool = False):
        self.bits, self.D, self.F, self.g = bits, D, F, g
        self.gate_up, self.down, self.raw = [], [], []
        for e in range(E):
            gt, u, d = workloads.moe_expert(e, D, F, stream)
            self.raw.append((gt, u, d))
            self.gate_up.append(GpuWeight(workloads.interleave_row_blocks(gt, u), bits, g=g, packed_zeros=packed_zeros))
            self.down.append(GpuWeight(d, bits, g=g, packed_zeros=packed_zeros))
        self._oracle = {}

    def oracle_expert(self, e):
        """The oracle's own quantization of expert e: (gate, up, down) dicts."""
        if e not in self._oracle:
            self._oracle[e] = tuple(oracle.quantize(m, self.bits, g=self.g) for m in self.raw[e])
        return self._oracle[e]

    def oracle_sets(self, used):
        gs, us, ds = [], [], []
        for e, (g, u, d) in enumerate(self.raw):
            if e in used:
                a, b, c = self.oracle_expert(e)
            else:  # never referenced by the tokens passed to the oracle
                z = lambda n, k: dict(codes=np.zeros((n, k), np.uint8), scales=np.zeros((n, k // self.g), np.uint16),
                                      zeros=np.zeros((n, k // self.g), np.uint8), g=self.g)
                a, b, c = z(*g.shape), z(*u.shape), z(*d.shape)
            gs.append(a)
            us.append(b)
            ds.append(c)
        return gs, us, ds


def dequant(qd):
    g = qd.get("g", 128)
    s = qd["scales"].view(np.float16).astype(np.float64)
    z = qd["zeros"].astype(np.float64)
    return (qd["codes"] - np.repeat(z, g, 1)) * np.repeat(s, g, 1)


def near_tie(v, abs_err=0.0):
    """(fp16 rounding of v, its ulp, mask of elements whose exact value lies within
    ulp/256 + abs_err of a rounding midpoint)."""
    a16 = v.astype(np.float16)
    ulp = np.spacing(np.abs(a16)).astype(np.float64)
    dist = ulp / 2 - np.abs(v - a16.astype(np.float64))
    return a16, ulp, dist <= ulp / 256 + abs_err


def swiglu_abs_err(x_row, g: dict, u: dict):
    """Bound on the fp32 error of silu(g)*u as the GPU forms it: g and u each pass through a
    few dozen fp32 roundings (matrix-core accumulation per 32 k, one fma per 128-k group),
    each at most 2^-24 of sum_k |x_k w_k|; silu' <= 1.1.  64 roundings are allowed."""
    xa = np.abs(x_row.astype(np.float64))
    Ag, Au = np.abs(dequant(g)) @ xa, np.abs(dequant(u)) @ xa
    gv, uv = oracle.linear(x_row[None], g)[0], oracle.linear(x_row[None], u)[0]
    silu = gv / (1 + np.exp(-gv))
    return 64 * 2.0 ** -24 * (1.1 * np.abs(uv) * Ag + np.abs(silu) * Au)


def flip_bound(ex: Experts, x, ids, wts):
    """Per-output worst-case effect of near-tie intermediate elements rounding the other way."""
    T, K = ids.shape
    bound = np.zeros((T, ex.D))
    for t in range(T):
        for j in range(K):
            e = int(ids[t, j])
            g, u, d = ex.oracle_expert(e)
            v = oracle.swiglu_act(x[t], g, u)
            _, ulp, near = near_tie(v)
            if near.any():
                cols = np.nonzero(near)[0]
                gd = d.get("g", 128)
                wd = (d["codes"][:, cols].astype(np.float64) - d["zeros"][:, cols // gd]) * \
                    d["scales"][:, cols // gd].view(np.float16).astype(np.float64)
                bound[t] += float(wts[t, j]) * (np.abs(wd) * ulp[cols]).sum(axis=1)
    return bound


def check_ffn(y, r, bound):
    rms = np.sqrt(np.mean(r * r))
    allowed = TOL * np.maximum(np.abs(r), 0.01 * rms) + bound
    excess = np.abs(y.astype(np.float64) - r) - allowed
    assert (excess <= 0).all(), report(y, r) + f" worst_excess={excess.max():.3e} flips_allowed_at={int((bound > 0).sum())}"


def run_ffn(ex: Experts, x, ids, wts):
    torch, q = gpu()
    T, D = x.shape
    K = ids.shape[1]
    E, F = len(ex.down), ex.F
    ws_bytes = q.qmoe_ffn_workspace_bytes(T, K, E, D, F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    q.qmoe_ffn(ex.gate_up[0].desc, [g.handle() for g in ex.gate_up], ex.down[0].desc, [g.handle() for g in ex.down],
               to_dev_fp16(x), D, T, dev(ids), dev(wts), K, out, D, ws, ws_bytes)
    torch.cuda.synchronize()
    return from_dev_fp16(out)


def small_routing(T, E, seed):
    ids, wts = workloads.zipf_routing(T, E, 2, 1.1, seed)
    ids[ids == 3] = 2            # expert 3 receives no rows
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], 4, ids[:, 1])
    ids[:, 0] = np.where(ids[:, 1] == ids[:, 0], 0, ids[:, 0])
    assert np.bincount(ids.ravel(), minlength=E)[3] == 0
    return ids, wts


@pytest.mark.parametrize("bits", (4, 2, 6))
def test_grouped_projections_parity(bits):
    """Each grouped projection at the standard tolerance: gate/up (fp32 rows and fp16 rows)
    on gathered token rows, down on the oracle's fp16 intermediate."""
    torch, q = gpu()
    E, D, F, T = 5, 512, 768, 37
    ex = Experts(E, D, F, bits, stream=50 + bits)
    x = workloads.activations_fp16(T, D, 51)
    ids, wts = small_routing(T, E, 52)
    order, offsets, row_src, _ = expected_dispatch(ids, E)
    R = len(order)
    xd, off_d, src_d = to_dev_fp16(x), dev(offsets), dev(row_src)

    y32 = torch.empty((R, 2 * F), dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ex.gate_up[0].desc, [g.handle() for g in ex.gate_up], xd, D, src_d, off_d, R,
                           q.QP_EPI_ROWS_F32, y32, 2 * F)
    y16 = torch.empty((R, 2 * F), dtype=torch.int16, device="cuda")
    q.qlinear_grouped_gemm(ex.gate_up[0].desc, [g.handle() for g in ex.gate_up], xd, D, src_d, off_d, R,
                           q.QP_EPI_NONE, y16, 2 * F)
    torch.cuda.synchronize()
    y32, y16 = y32.cpu().numpy(), from_dev_fp16(y16)
    a_ref = np.zeros((R, F), np.float16)
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows) == 0:
            continue
        g, u, _ = ex.oracle_expert(e)
        gu = oracle.quantize(workloads.interleave_row_blocks(*ex.raw[e][:2]), bits)
        r = oracle.linear(x[row_src[rows]], gu)
        assert rel_err(y32[rows], r) <= TOL, (e, report(y32[rows], r))
        assert rel_err(y16[rows], r) <= TOL, (e, report(y16[rows], r))
        for i, row in enumerate(rows):
            a_ref[row] = oracle.swiglu_act(x[row_src[row]], g, u).astype(np.float16)

    # down projection on the oracle's intermediate, fp32 rows
    yd = torch.empty((R, D), dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ex.down[0].desc, [g.handle() for g in ex.down], to_dev_fp16(a_ref), F, None, off_d, R,
                           q.QP_EPI_ROWS_F32, yd, D)
    torch.cuda.synchronize()
    yd = yd.cpu().numpy()
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows):
            r = oracle.linear(a_ref[rows], ex.oracle_expert(e)[2])
            assert rel_err(yd[rows], r) <= TOL, (e, report(yd[rows], r))


@pytest.mark.parametrize("sizes,base,slack", (([70, 33, 32, 1, 0, 15, 16, 17], 0, 0),
                                                ([150, 129, 0, 5], 0, 0),
                                                ([0, 0, 0, 0, 0, 0, 0, 97], 0, 0),
                                                ([40, 0, 31, 9], 7, 50)),
                         ids=("small-geometry", "layer-geometry", "last-expert-only", "offset-base-and-slack"))
def test_grouped_row_tiles(sizes, base, slack):
    """Expert row counts at and around the 32- and 128-row tile edges, on both workgroup
    geometries (at most 32 rows per expert on average selects the 4-wave, 32-row one); all
    rows on the last expert; and a routing that starts at sorted row `base` under a row
    bound `slack` rows above its end (rows outside the routing stay untouched)."""
    torch, q = gpu()
    E, D, N = len(sizes), 256, 512
    offsets = (base + np.concatenate([[0], np.cumsum(sizes)])).astype(np.int32)
    R = int(offsets[-1]) + slack
    x = workloads.activations_fp16(R, D, 71)
    raw = [workloads.weights_fp16(N, D, 700 + e) for e in range(E)]
    ws = [GpuWeight(w, 4) for w in raw]
    y = torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ws[0].desc, [w.handle() for w in ws], to_dev_fp16(x), D, None, dev(offsets), R,
                           q.QP_EPI_ROWS_F32, y, N)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows):
            r = oracle.linear(x[rows], oracle.quantize(raw[e], 4))
            assert rel_err(y[rows], r) <= TOL, (e, report(y[rows], r))
    outside = np.r_[0:offsets[0], offsets[-1]:R]
    assert np.all(y[outside] == 7.0)


def test_grouped_64_experts():
    """The most experts one launch takes: every lane of the work-item scan holds an expert,
    with empty experts, a large one and single rows spread over the table."""
    torch, q = gpu()
    E, D, N = 64, 256, 256
    rng = np.random.default_rng(7300)
    sizes = rng.integers(0, 6, E)
    sizes[[0, 13, 63]] = [0, 75, 33]
    sizes[rng.choice(E, 8, replace=False)] = 0
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    x = workloads.activations_fp16(R, D, 73)
    raw = [workloads.weights_fp16(N, D, 7300 + e) for e in range(E)]
    ws = [GpuWeight(w, 3) for w in raw]
    y = torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")
    q.qlinear_grouped_gemm(ws[0].desc, [w.handle() for w in ws], to_dev_fp16(x), D, None, dev(offsets), R,
                           q.QP_EPI_ROWS_F32, y, N)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if len(rows):
            r = oracle.linear(x[rows], oracle.quantize(raw[e], 3))
            assert rel_err(y[rows], r) <= TOL, (e, report(y[rows], r))


@pytest.mark.parametrize("bits", (4, 2))
def test_swiglu_epilogue_rounding(bits):
    """The SwiGLU epilogue's fp16 result equals the oracle's rounding of silu(g)*u except
    at near-ties, where it may be the other neighbour (never more than one ulp)."""
    torch, q = gpu()
    E, D, F, T = 4, 512, 512, 40
    ex = Experts(E, D, F, bits, stream=70 + bits)
    x = workloads.activations_fp16(T, D, 71)
    ids, _ = workloads.zipf_routing(T, E, 2, 1.1, 72)
    order, offsets, row_src, _ = expected_dispatch(ids, E)
    R = len(order)
    a = torch.empty((R, F), dtype=torch.int16, device="cuda")
    q.qlinear_grouped_gemm(ex.gate_up[0].desc, [g.handle() for g in ex.gate_up], to_dev_fp16(x), D,
                           dev(row_src), dev(offsets), R, q.QP_EPI_SWIGLU, a, F)
    torch.cuda.synchronize()
    a = from_dev_fp16(a)
    mism = 0
    for e in range(E):
        g, u, _ = ex.oracle_expert(e)
        for row in range(offsets[e], offsets[e + 1]):
            v = oracle.swiglu_act(x[row_src[row]], g, u)
            a16, ulp, near = near_tie(v, swiglu_abs_err(x[row_src[row]], g, u))
            diff = a[row] != a16
            assert not (diff & ~near).any(), (e, row, np.nonzero(diff & ~near)[0][:5])
            assert (np.abs(a[row].astype(np.float64) - a16) <= ulp * 1.0001).all()
            mism += int(diff.sum())
    assert mism <= R * F // 100


@pytest.mark.parametrize("bits", (4, 2, 6))
@pytest.mark.parametrize("F", (768, 1024), ids=("down-one-pass", "down-two-k-halves"))
def test_moe_ffn_small(bits, F):
    """d_ff = 768 runs the down projection in one pass, 1024 in two k halves summed by the
    combine."""
    E, D, T = 5, 512, 37
    ex = Experts(E, D, F, bits, stream=50 + bits)
    x = workloads.activations_fp16(T, D, 51)
    ids, wts = small_routing(T, E, 52)
    y = run_ffn(ex, x, ids, wts)
    r = oracle.moe_ffn(x, ids, wts, *ex.oracle_sets(set(range(E))))
    check_ffn(y, r, flip_bound(ex, x, ids, wts))


def test_moe_all_tokens_one_expert_many_tiles():
    """130 rows on one expert: more than the 128-row pass of the grouped kernel."""
    E, D, F, T = 2, 256, 512, 130
    ex = Experts(E, D, F, 4, stream=60)
    x = workloads.activations_fp16(T, D, 61)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    y = run_ffn(ex, x, ids, wts)
    r = oracle.moe_ffn(x, ids, wts, *ex.oracle_sets({0}))
    check_ffn(y, r, flip_bound(ex, x, ids, wts))


@pytest.mark.timeout(900)
def test_moe_ffn_full_sampled():
    """16 experts, d_model 4096, d_ff 14336, 128 tokens top-2 Zipf(1.1): the whole FFN on the
    GPU in the launch sequence the benchmark uses; at least 16 tokens, chosen so that together
    they route to every active expert, recomputed by the oracle."""
    E, D, F = workloads.MOE_EXPERTS, workloads.MOE_DMODEL, workloads.MOE_DFF
    x, ids, wts = workloads.moe_inputs()
    ex = Experts(E, D, F, 4, stream=5)
    y = run_ffn(ex, x, ids, wts)
    assert np.isfinite(y).all()
    chosen = [0, 5, 77, 127]
    for e in np.unique(ids):
        if e not in ids[chosen]:
            chosen.append(int(np.nonzero((ids == e).any(axis=1))[0][0]))
    for t in np.linspace(0, len(ids) - 1, 16).astype(int):
        if len(chosen) >= 16:
            break
        if t not in chosen:
            chosen.append(int(t))
    pick = np.array(sorted(chosen))
    assert len(pick) >= 16 and set(ids[pick].ravel()) == set(np.unique(ids))
    print(f"moe full: {len(pick)} tokens cover {len(np.unique(ids))} active experts", flush=True)
    used = set(ids[pick].ravel().tolist())
    r = oracle.moe_ffn(x[pick], ids[pick], wts[pick], *ex.oracle_sets(used))
    check_ffn(y[pick], r, flip_bound(ex, x[pick], ids[pick], wts[pick]))
