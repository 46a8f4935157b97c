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


def _expert(entries, n, k, zp=8):
    """A 4-bit expert matrix [n, k] whose dequantized weights are 0 except `entries`
    {(row, col): small integer}: scale 1.0, zero point 8, so code = value + 8."""
    codes = np.full((n, k), zp, np.uint8)
    for (i, j), v in entries.items():
        codes[i, j] = zp + v
    G = k // 128
    return dict(codes=codes, scales=np.full((n, G), np.float16(1.0)).view(np.uint16),
                zeros=np.full((n, G), zp, np.uint8), g=128)


def test_hand_worked_two_expert_swiglu():
    """One token x = e_0 routed to two experts with combine weights 0.75 and 0.125 (not
    summing to 1: the oracle must use the weights it is given, not renormalise them).

    Expert 0: gate[0,0] = 2, up[0,0] = 3  -> a_0 = fp16(silu(2) * 3)
      silu(2) * 3 = 6 / (1 + e^-2) = 6 / 1.1353352832... = 5.2847824678...
      fp16 spacing on [4, 8) is 2^-8: 5.28478... * 256 = 1352.90 -> 1353 / 256 = 5.28515625
      down[0,0] = 1, down[1,0] = -2   -> o = (5.28515625, -10.5703125, 0, ...)
    Expert 1: gate[0,0] = -1, up[0,0] = 4 -> a_0 = fp16(silu(-1) * 4)
      silu(-1) * 4 = -4 / (1 + e) = -4 / 3.7182818284... = -1.0757656854...
      fp16 spacing on [1, 2) is 2^-10: -1101.58 -> -1102 / 1024 = -1.076171875
      down[0,0] = 3, down[1,0] = 1    -> o = (-3.228515625, -1.076171875, 0, ...)
    out[0] = 0.75 * 5.28515625 + 0.125 * -3.228515625 = 3.9638671875 - 0.403564453125 = 3.560302734375
    out[1] = 0.75 * -10.5703125 + 0.125 * -1.076171875 = -7.927734375 - 0.134521484375 = -8.062255859375
    Every other output is 0.  All these values are dyadic, so the fp64 result is exact."""
    D = F = 128
    gate = [_expert({(0, 0): 2}, F, D), _expert({(0, 0): -1}, F, D)]
    up = [_expert({(0, 0): 3}, F, D), _expert({(0, 0): 4}, F, D)]
    down = [_expert({(0, 0): 1, (1, 0): -2}, D, F), _expert({(0, 0): 3, (1, 0): 1}, D, F)]
    x = np.zeros((1, D), np.float16)
    x[0, 0] = 1.0
    ids = np.array([[0, 1]], np.int32)
    wts = np.array([[0.75, 0.125]], np.float32)
    r = oracle.moe_ffn(x, ids, wts, gate, up, down)
    want = np.zeros(D)
    want[0], want[1] = 3.560302734375, -8.062255859375
    assert np.array_equal(r[0], want)
    # the SwiGLU intermediate before its fp16 rounding
    v = oracle.swiglu_act(x[0], gate[0], up[0])
    assert abs(v[0] - 5.2847824678672947) < 1e-12 and not v[1:].any()


def test_all_rows_to_one_expert_equals_dense_ffn_from_linear():
    """Every token routed to expert 1 with weight 1 (top-1): the FFN equals the dense
    chain built from the oracle's linear layer, down(fp16(silu(gate x) * (up x)))."""
    g, u, d = experts(4)
    x = workloads.activations_fp16(5, D, 4)
    ids = np.ones((5, 1), np.int32)
    wts = np.ones((5, 1), np.float32)
    got = oracle.moe_ffn(x, ids, wts, g, u, d)
    gv, uv = oracle.linear(x, g[1]), oracle.linear(x, u[1])
    a = (gv / (1.0 + np.exp(-gv)) * uv).astype(np.float16)
    want = oracle.linear(a, d[1])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
