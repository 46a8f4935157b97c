"""Pins for the oracle's routed-expert FFN (on-device MoE page, s4.2: tasks carry the
hidden states and the top-k expert ids; the experts are gate/up/down FFNs)."""
import numpy as np

import oracle
import workloads

D, F, E = 256, 384, 3


def experts(seed):
    mk = lambda n, k, s: oracle.quantize(workloads.weights_fp16(n, k, s), 4)
    return ([mk(F, D, seed + 10 * e) for e in range(E)],
            [mk(F, D, seed + 10 * e + 1) for e in range(E)],
            [mk(D, F, seed + 10 * e + 2) for e in range(E)])


def dq(q):
    s = q["scales"].view(np.float16).astype(np.float64)
    z = q["zeros"].astype(np.float64)
    return (q["codes"] - np.repeat(z, 128, 1)) * np.repeat(s, 128, 1)


def test_single_expert_reduces_to_dense_ffn():
    """topk = 1, weight 1: out = Wd * fp16(silu(Wg x) * (Wu x)), all via numpy fp64
    matmuls and numpy's RNE fp16 cast."""
    g, u, d = experts(1)
    x = workloads.activations_fp16(4, D, 1)
    ids = np.array([[2], [0], [1], [2]], np.int32)
    wts = np.ones((4, 1), np.float32)
    got = oracle.moe_ffn(x, ids, wts, g, u, d)
    xf = x.astype(np.float64)
    for t in range(4):
        e = ids[t, 0]
        gv, uv = dq(g[e]) @ xf[t], dq(u[e]) @ xf[t]
        a = (gv / (1 + np.exp(-gv)) * uv).astype(np.float16).astype(np.float64)
        assert np.allclose(got[t], dq(d[e]) @ a, rtol=1e-12, atol=1e-13)


def test_top2_is_weighted_sum_and_token_order_free():
    g, u, d = experts(2)
    x = workloads.activations_fp16(6, D, 2)
    ids, wts = workloads.zipf_routing(6, E, 2, 1.1, 3)
    both = oracle.moe_ffn(x, ids, wts, g, u, d)
    first = oracle.moe_ffn(x, ids[:, :1], wts[:, :1], g, u, d)
    second = oracle.moe_ffn(x, ids[:, 1:], wts[:, 1:], g, u, d)
    assert np.allclose(both, first + second, rtol=1e-12, atol=1e-14)
    perm = np.array([4, 1, 5, 0, 3, 2])
    shuffled = oracle.moe_ffn(x[perm], ids[perm], wts[perm], g, u, d)
    assert np.array_equal(shuffled, both[perm])
    # linear in the combine weight
    half = oracle.moe_ffn(x, ids, wts * np.float32(0.5), g, u, d)
    assert np.allclose(half, 0.5 * both, rtol=1e-12, atol=1e-14)


def test_zipf_routing_skew():
    """Popularity skew of the MoE page, s1.3: about 80% of tokens land on half of the
    experts.  Zipf(1.1) over 16 experts puts ~83% of the mass on the top 8."""
    ids, wts = workloads.zipf_routing(20000, 16, 2, 1.1, 9)
    share = np.isin(ids, np.arange(8)).mean()
    assert 0.75 < share < 0.88
    assert (wts > 0).all() and (wts.sum(1) <= 1.0 + 1e-6).all()
    assert (ids[:, 0] != ids[:, 1]).all()
