"""Pins for the oracle's fp8 block scales with an fp16 fallback (mixed-bit page, s2.3: 8-bit
float scales bring 2-bit groups of 32 to 2.25 bits per weight; the few blocks out of the fp8
range keep fp16 scales).  The E4M3 decoder is checked against torch's float8_e4m3fn on all 256
codes; the rounding-up encoder against torch's round-to-nearest conversion; the row quantizer
on a hand-worked row, against the fp16-path quantizer on its fallback groups, and by
invariants; the storage against the page's 2.25 bits per weight."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def test_e4m3_values_match_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0 and got[0x78] == 256.0


def test_e4m3_ceil_is_the_smallest_code_not_below_t():
    rng = np.random.default_rng(3)
    ts = np.concatenate([2.0 ** rng.uniform(-6, np.log2(448), 4000), [2.0 ** -6, 1.0, 256.0, 448.0, 1.0001, 447.9]])
    for t in ts.astype(np.float32):
        c = oracle.e4m3_ceil(float(t))
        v = oracle.e4m3_value(c)
        assert v >= t and (c == 0x01 or oracle.e4m3_value(c - 1) < t), (t, c)
        # torch rounds to nearest: the ceiling is that value or the next code up
        rn = torch.tensor([float(t)], dtype=torch.float32).to(torch.float8_e4m3fn)
        rc = int(rn.view(torch.uint8).item())
        assert c in (rc, rc + 1), (t, c, rc)
    assert oracle.e4m3_ceil(449.0) == -1


def test_hand_row_symmetric_two_bit():
    # g = 32, 2 bits, symmetric (qmax 3, midpoint 2).  Group 0: max |w| 0.75 -> s32 = 1.5/3 = 0.5
    # is the row maximum, F = 0.5 * 2^-8 = 2^-9, t = 256 -> code 0x78, stored 0.5.  Group 1:
    # max 0.25 -> s32 = 0.5/3 (fp32 0.16666667), t = 85.33 -> smallest E4M3 >= t is 88
    # (1.375 * 2^6: exponent field 6 + 7 = 13, mantissa 3, code 0x6B), stored 88 * 2^-9 = 0.171875.  Group 2: max 2^-20 ->
    # s32 = 2^-19/3, t = 2^-10/3 < 2^-6 -> fp16 fallback 2^-14 (the fp16 path's floor), code
    # 0x80 (first fallback).  Group 3: all zero -> code 0, codes at the midpoint.
    w = np.zeros((1, 128), np.float16)
    w[0, 0], w[0, 1], w[0, 2] = 0.75, -0.5, 0.125
    w[0, 32], w[0, 33], w[0, 34] = 0.25, -0.25, 0.0859375
    w[0, 64] = 2.0 ** -20
    q = oracle.quantize_fp8(w, 2, 32, sym=True)
    assert q["factors"][0] == np.float32(2.0 ** -9)
    assert list(q["sc8"][0]) == [0x78, 0x6B, 0x80, 0x00]
    assert q["scales_f32"][0, 0] == 0.5 and q["scales_f32"][0, 1] == 0.171875
    assert q["fb"][0, 0] == 0x0400 and q["counts"][0] == 1
    # codes: rint(w / s) + 2 clamped to [0, 3]: 0.75/0.5 = 1.5 -> 2 (even) -> 4 -> 3;
    # -0.5/0.5 = -1 -> 1; 0.125/0.5 = 0.25 -> 0 -> 2; 0.25/0.171875 = 1.4545 -> 1 -> 3;
    # -1.4545 -> -1 -> 1; 0.0859375/0.171875 = 0.5 -> 0 (even) -> 2
    assert list(q["codes"][0, :3]) == [3, 1, 2] and list(q["codes"][0, 32:35]) == [3, 1, 2]
    assert (q["codes"][0, 96:] == 2).all() and q["zeros"][0, 3] == 2


def test_fallback_groups_equal_the_fp16_path():
    """Groups planted far below the row's largest scale fall back; their scale, zero point
    and codes are the fp16 path's (or_quantize_group), in row order of the fallback list."""
    rng = np.random.default_rng(11)
    for sym in (False, True):
        w = workloads.weights_fp16(6, 512, 40 + sym)
        w[:, :32] *= np.float16(40.0)                    # a large group sets each row's factor
        tiny = [(0, 3), (0, 9), (2, 5), (5, 15)]
        for r, gi in tiny:
            w[r, 32 * gi:32 * gi + 32] = (rng.standard_normal(32) * 2e-6).astype(np.float16)
        q = oracle.quantize_fp8(w, 3, 32, sym=sym)
        assert int(q["counts"].sum()) == len(tiny)
        for r in range(6):
            seen = 0
            for gi in range(16):
                c = q["sc8"][r, gi]
                if (r, gi) in tiny:
                    assert c == 0x80 | seen
                    grp = w[r, 32 * gi:32 * gi + 32]
                    if sym:
                        sh, codes = oracle.quantize_group_sym(grp, 3)
                    else:
                        sh, zp, codes = oracle.quantize_group(grp, 3)
                        assert q["zeros"][r, gi] == zp
                    assert q["fb"][r, seen] == sh
                    assert np.array_equal(q["codes"][r, 32 * gi:32 * gi + 32], codes)
                    seen += 1
                else:
                    assert c < 0x80


@pytest.mark.parametrize("bits,g,sym", ((2, 32, True), (4, 128, False), (3, 64, False), (6, 32, True), (5, 64, True)))
def test_invariants_on_layer_rows(bits, g, sym):
    w = workloads.weights_fp16(64, 4096, 50 + bits)
    q = oracle.quantize_fp8(w, bits, g, sym=sym)
    qmax = (1 << bits) - 1
    assert q["codes"].max() <= qmax and int(q["counts"].sum()) == 0
    # every stored scale is F times an E4M3 value of at most 256, and covers the group's range
    G = 4096 // g
    for r in range(64):
        F = float(q["factors"][r])
        for gi in range(G):
            c = int(q["sc8"][r, gi])
            assert 0 < c <= 0x78
            assert q["scales_f32"][r, gi] == np.float32(F * oracle.e4m3_value(c))
    # Error bound: half a step, plus the top-code clamp when the stored scale sits below the
    # exact range / qmax (only by an fp32 rounding: the E4M3 value rounds up; it happens on each
    # row's largest group, whose stored scale is its own fp32 scale).
    wf = w.astype(np.float64).reshape(64, G, g)
    rng_ = np.abs(wf).max(2) * 2 if sym else np.maximum(wf.max(2), 0) - np.minimum(wf.min(2), 0)
    sc = q["scales_f32"].astype(np.float64)
    # + the fp32 rounding of the quotient w / s (at most qmax * 2^-24 steps) at a tie
    bound = sc / 2 + qmax * np.maximum(rng_ / qmax - sc, 0) + (qmax + 1) * 2.0 ** -23 * sc + 1e-12
    err = np.abs(wf - oracle.dequant_fp8(q).reshape(64, G, g)).max(2)
    assert (err <= bound).all()
    assert (rng_ / qmax - sc <= sc * 2 ** -22).all()  # below the exact scale by at most a rounding


def test_storage_is_two_and_a_quarter_bits_per_weight():
    """2-bit symmetric groups of 32 with fp8 scales: 2 + 8/32 = 2.25 bits per weight (the
    page's figure), plus one fp32 row factor (32/K bits)."""
    N, K = 64, 4096
    q = oracle.quantize_fp8(workloads.weights_fp16(N, K, 60), 2, 32, sym=True)
    stored = N * K * 2 // 8 + q["sc8"].nbytes + q["factors"].nbytes
    assert q["sc8"].nbytes == N * K // 32
    assert 8 * stored / (N * K) == 2.25 + 32 / K
    assert oracle.quant_bytes(N * K, 2, 32, 1, 0) * 8 / (N * K) == 2.25


def test_all_zero_rows_and_groups():
    w = np.zeros((2, 256), np.float16)
    w[1, 200] = 0.5
    for sym in (False, True):
        q = oracle.quantize_fp8(w, 4, 64, sym=sym)
        assert q["factors"][0] == 1.0 and not q["sc8"][0].any() and q["counts"].sum() == 0
        mid = 8 if sym else 0
        assert (q["codes"][0] == mid).all() and (q["codes"][1, :192] == mid).all()
        assert list(q["sc8"][1, :3]) == [0, 0, 0] and q["sc8"][1, 3] == 0x78


def test_moe_ffn_fp8_equals_the_fp16_ffn_on_equal_scales():
    """The fp8-scale expert FFN (numpy) against the C oracle's FFN: with every stored scale an
    fp16 value (the fp16 path's own quantization, its scales carried as fp32), both compute
    the same definition, so the two agree to fp64 rounding."""
    E, D, F, T = 3, 128, 256, 6
    x = workloads.activations_fp16(T, D, 70)
    ids = np.array([[0, 2], [1, 0], [2, 1], [2, 0], [0, 1], [1, 2]], np.int32)
    wts = np.array([[0.7, 0.3], [0.5, 0.25], [1.0, 0.125], [0.6, 0.4], [0.9, 0.1], [0.2, 0.8]], np.float32)
    q16 = [[oracle.quantize(m, 4) for m in workloads.moe_expert(e, D, F, 71)] for e in range(E)]
    as8 = lambda d: dict(codes=d["codes"], zeros=d["zeros"], g=128,
                         scales_f32=d["scales"].view(np.float16).astype(np.float32))
    r16 = oracle.moe_ffn(x, ids, wts, *[[q16[e][i] for e in range(E)] for i in range(3)])
    r8 = oracle.moe_ffn_fp8(x, ids, wts, *[[as8(q16[e][i]) for e in range(E)] for i in range(3)])
    rms = np.sqrt(np.mean(r16 * r16))
    assert rms > 0 and np.abs(r8 - r16).max() <= 1e-12 * rms
    # one token through one expert with weight 1 is silu(gate) * up rounded to fp16, then down
    g, u, dn = (as8(d) for d in q16[1])
    a = oracle.swiglu_act_fp8(x[:1], g, u).astype(np.float16)
    one = oracle.moe_ffn_fp8(x[:1], np.array([[1]], np.int32), np.array([[1.0]], np.float32), [g] * E, [u] * E, [dn] * E)
    assert np.array_equal(one, oracle.linear_fp8(a, dn))


def test_linear_a8_fp8_equals_the_c_integer_dot_on_equal_scales():
    """The int8-activation product over fp8-scale weights (numpy) against the C oracle's
    integer-dot product when every stored scale is an fp16 value: same definition, same
    integer group sums, so the two agree to fp64 rounding."""
    w = workloads.weights_fp16(48, 512, 80)
    x = workloads.activations_fp16(5, 512, 81)
    xq, sx = oracle.act_quantize(x)
    q16 = oracle.quantize(w, 3)
    as8 = dict(codes=q16["codes"], zeros=q16["zeros"], g=128, scales_f32=q16["scales"].view(np.float16).astype(np.float32))
    r16 = oracle.linear_a8(xq, sx, q16)
    r8 = oracle.linear_a8_fp8(xq, sx, as8)
    assert np.abs(r8 - r16).max() <= 1e-12 * np.abs(r16).max()
