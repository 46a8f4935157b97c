"""GPU parity for the routed-expert path: dispatch (bit-exact integer work), the grouped
GEMM epilogues, and the whole FFN (qmoe_ffn) against the oracle's fp64 routed FFN."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu


def test_dispatch_exact():
    torch, q = gpu()
    T, E, K = 300, 12, 2
    ids, wts = workloads.zipf_routing(T, E, K, 1.1, 77)
    ids[ids == 5] = 4  # leave expert 5 empty
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % E, ids[:, 1])
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")              # stable in (token, choice) order
    want_off = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))])
    want_src = order // K
    want_rows = np.empty(T * K, np.int64)
    want_rows[order] = np.arange(T * K)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
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
    """Gate/up interleaved by 16-row blocks and down, quantized and packed on the GPU."""

    def __init__(self, E, D, F, bits, config):
        self.gate_up, self.down, self.raw = [], [], []
        for e in range(E):
            g, u, d = workloads.moe_expert(e, D, F, config)
            self.raw.append((g, u, d))
            self.gate_up.append(GpuWeight(workloads.interleave_row_blocks(g, u), bits))
            self.down.append(GpuWeight(d, bits))

    def oracle_sets(self, bits, used):
        gs, us, ds = [], [], []
        for e, (g, u, d) in enumerate(self.raw):
            if e in used:
                gs.append(oracle.quantize(g, bits))
                us.append(oracle.quantize(u, bits))
                ds.append(oracle.quantize(d, bits))
            else:  # never referenced by the sampled tokens: zero placeholders
                z = lambda n, k: dict(codes=np.zeros((n, k), np.uint8), scales=np.zeros((n, k // 128), np.uint16),
                                      zeros=np.zeros((n, k // 128), np.uint8))
                gs.append(z(*g.shape))
                us.append(z(*u.shape))
                ds.append(z(*d.shape))
        return gs, us, ds


def run_ffn(ex: Experts, x, ids, wts):
    torch, q = gpu()
    T, D = x.shape
    K = ids.shape[1]
    E = len(ex.down)
    F = ex.down[0].k
    d_gu, d_dn = ex.gate_up[0].desc, ex.down[0].desc
    ws_bytes = q.qmoe_ffn_workspace_bytes(T, K, E, D, F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q.qmoe_ffn(d_gu, [g.handle() for g in ex.gate_up], d_dn, [g.handle() for g in ex.down], to_dev_fp16(x), D, T,
               dev(ids), dev(wts), K, out, D, ws, ws_bytes)
    torch.cuda.synchronize()
    return from_dev_fp16(out)


@pytest.mark.parametrize("bits", (4, 2, 6))
def test_moe_ffn_small(bits):
    E, D, F, T = 5, 512, 768, 37
    ex = Experts(E, D, F, bits, config=50 + bits)
    x = workloads.activations_fp16(T, D, 51)
    ids, wts = workloads.zipf_routing(T, E, 2, 1.1, 52)
    ids[ids == 3] = 2            # expert 3 receives no rows
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], 4, ids[:, 1])
    ids[:, 0] = np.where(ids[:, 1] == ids[:, 0], 0, ids[:, 0])
    assert (np.bincount(ids.ravel(), minlength=E)[3] == 0)
    y = run_ffn(ex, x, ids, wts)
    r = oracle.moe_ffn(x, ids, wts, *ex.oracle_sets(bits, set(range(E))))
    assert rel_err(y, r) <= TOL, report(y, r)


def test_moe_all_tokens_one_expert_many_tiles():
    """130 rows on one expert: more than the 128-row tile of the grouped kernel."""
    E, D, F, T = 2, 256, 512, 130
    ex = Experts(E, D, F, 4, config=60)
    x = workloads.activations_fp16(T, D, 61)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    y = run_ffn(ex, x, ids, wts)
    r = oracle.moe_ffn(x, ids, wts, *ex.oracle_sets(4, {0}))
    assert rel_err(y, r) <= TOL, report(y, r)


def test_moe_config_full_sampled():
    """16 experts, d_model 4096, d_ff 14336, 128 tokens top-2 Zipf(1.1): the whole FFN on the
    GPU, 4 tokens recomputed by the oracle."""
    E, D, F = workloads.MOE_EXPERTS, workloads.MOE_DMODEL, workloads.MOE_DFF
    x, ids, wts = workloads.moe_inputs()
    ex = Experts(E, D, F, 4, config=5)
    y = run_ffn(ex, x, ids, wts)
    assert np.isfinite(y).all()
    pick = np.array([0, 5, 77, 127])
    used = set(ids[pick].ravel().tolist())
    r = oracle.moe_ffn(x[pick], ids[pick], wts[pick], *ex.oracle_sets(4, used))
    assert rel_err(y[pick], r) <= TOL, report(y[pick], r)
