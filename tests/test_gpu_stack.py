"""GPU parity for the Llama-7B-shaped decode stack at M = 1 at its real shapes and bit widths:
each distinct layer type of the mixed bit table runs through the same four qlinear_gemv_batch
stages the benchmark times ([q, k, v], [o], [gate, up], [down]), and every output is compared
with the oracle's fp64 linear layer within the floored relative tolerance.

Layer types (mixed-bit page, s2.2: per-projection bit mix): layers 0 and 31 all 6-bit;
layers 1-21 q/k 2-bit, v 6, o 5, gate/up 2, down 5; layers 22-30 the same with q/k 3-bit.
The [gate, up] stage is 2 x 11008 rows at 2 bits in one launch, [down] 4096 x 11008 at 5 bits."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, GpuWeight, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu

STAGES = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("layer", (0, 5, 25, 31))
def test_stack_layer_full_shapes(layer):
    torch, q = gpu()
    mats = {}
    for name in workloads.LLAMA_MATRICES:
        n, k = workloads.STACK_SHAPES[name]
        w = workloads.weights_fp16(n, k, workloads.stack_matrix_seed(layer, name))
        mats[name] = (w, workloads.stack_bits(layer, name))
    print(f"stack layer {layer}: bits " + " ".join(f"{nm}={b}" for nm, (_, b) in mats.items()), flush=True)
    xs = {k: workloads.activations_fp16(1, k, workloads.seed_for(3)) for k in (4096, 11008)}
    xd = {k: to_dev_fp16(v) for k, v in xs.items()}
    gws = {name: GpuWeight(w, b) for name, (w, b) in mats.items()}
    ys = {name: torch.empty((1, g.n), dtype=torch.int16, device="cuda") for name, g in gws.items()}
    for st in STAGES:
        probs = [q.gemv_problem(gws[nm].desc, gws[nm].handle(), xd[gws[nm].k], gws[nm].k, 1, ys[nm], gws[nm].n)
                 for nm in st]
        q.qlinear_gemv_batch(probs)
    torch.cuda.synchronize()
    for name, (w, b) in mats.items():
        ref = oracle.quantize(w, b)
        host = gws[name].host()
        assert np.array_equal(host["codes"], ref["codes"]), name
        r = oracle.linear(xs[w.shape[1]], ref)
        got = from_dev_fp16(ys[name])
        assert rel_err(got, r) <= TOL, (layer, name, b, report(got, r))
