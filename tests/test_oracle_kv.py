"""Pins for the oracle's quantized KV cache and decode attention (KV-cache quantization page,
kwkr.cn: s2.1 symmetric absmax scale, s2.2 groups along the head dimension, s2.3 K at INT4
with V at INT8, s3.1 FP32 scales, s5.1 two 4-bit values per byte and an operator that reads
the quantized cache directly).

The quantizer is pinned by what the page and arithmetic fix: codes in range, the absmax
element at +-qmax, the per-element error bound s/2, exact round-half-even ties on exactly
representable scales, the all-zero group.  The attention is pinned by closed forms (one
token, a zero query, two tokens), by token-order invariance and by a reduction to
scipy's softmax and numpy products on small inputs (GQA head mapping included).  The cache
layout is the library's own encoding: pinned by bijection, locality and round trips
(parity unpinned against the pages, which define no layout).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
D = oracle.KV_DIM


def _rows(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, D)) * scale).astype(np.float16)


def _deq(codes, scales, bits):
    g = D // scales.shape[1]
    q = codes.astype(np.int64) - (1 << (bits - 1))
    return q * np.repeat(scales.astype(np.float64), g, axis=1)


# ---- quantizer ------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantizer_range_and_absmax(bits, g):
    x = _rows(64, 11 + bits + g)
    codes, scales = oracle.kv_quantize(x, bits, g)
    qmax = (1 << (bits - 1)) - 1
    q = codes.astype(np.int64) - (1 << (bits - 1))
    assert q.min() >= -qmax and q.max() <= qmax
    xf = x.astype(np.float64).reshape(64, D // g, g)
    qg = q.reshape(64, D // g, g)
    for i in range(64):
        for j in range(D // g):
            m = np.abs(xf[i, j]).max()
            assert scales[i, j] == np.float32(np.float32(m) / np.float32(qmax))
            k = np.abs(xf[i, j]).argmax()
            assert abs(qg[i, j, k]) == qmax and np.sign(qg[i, j, k]) == np.sign(xf[i, j, k])


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantizer_error_bound(bits, g):
    """|x - q*s| <= s/2 + 2^-23 * m: rint's half step plus the fp32 rounding of x/s."""
    x = _rows(128, 5 * bits + g, scale=3.0)
    codes, scales = oracle.kv_quantize(x, bits, g)
    err = np.abs(x.astype(np.float64) - _deq(codes, scales, bits))
    s = np.repeat(scales.astype(np.float64), g, axis=1)
    m = np.repeat(np.abs(x.astype(np.float64)).reshape(128, D // g, g).max(axis=2), g, axis=1)
    assert (err <= s / 2 + 2.0 ** -23 * m).all()


def test_quantizer_ties_round_to_even():
    """m = 127/128 gives s = 2^-7 exactly at 8 bits, so x = (k + 1/2) * 2^-7 is an exact tie."""
    row = np.zeros(D, np.float16)
    row[0] = np.float16(127 / 128)
    halves = [0.5, 1.5, 2.5, 3.5, -2.5, -0.5, 126.5, -126.5]
    for i, h in enumerate(halves):
        row[1 + i] = np.float16(h / 128)
    codes, scales = oracle.kv_quantize(row[None], 8, 128)
    assert scales[0, 0] == np.float32(2.0 ** -7)
    q = codes[0].astype(int) - 128
    assert q[0] == 127
    assert list(q[1:1 + len(halves)]) == [0, 2, 2, 4, -2, 0, 126, -126]


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_zero_group(bits):
    x = _rows(2, 3)
    x[0, :64] = 0
    x[1, :] = np.float16(-0.0)
    codes, scales = oracle.kv_quantize(x, bits, 64)
    mid = 1 << (bits - 1)
    assert scales[0, 0] == 0 and (codes[0, :64] == mid).all() and scales[0, 1] > 0
    assert (scales[1] == 0).all() and (codes[1] == mid).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_constant_magnitude(bits):
    """A group of +-m maps to +-qmax exactly and dequantizes within one fp32 rounding."""
    qmax = (1 << (bits - 1)) - 1
    row = np.where(np.arange(D) % 3 == 0, -1.0, 1.0).astype(np.float16) * np.float16(0.7)
    codes, scales = oracle.kv_quantize(row[None], bits, 32)
    q = codes[0].astype(int) - (1 << (bits - 1))
    assert (np.abs(q) == qmax).all() and (np.sign(q) == np.sign(row.astype(float))).all()
    assert np.allclose(_deq(codes, scales, bits)[0], row.astype(np.float64), rtol=2.0 ** -23, atol=0)


def test_mixed_precision_bytes():
    """K at INT4 and V at INT8 for the page's 7B / 2048-token cache: 0.375 GB of data."""
    c = GOLD["kv_mixed_k4_v8"]
    rows = c["layers"] * c["kv_heads"] * c["tokens"]
    fp16 = oracle.kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"], 2)
    assert fp16 == c["fp16_bytes"]
    assert oracle.kv_cache_bytes(rows, c["k_bits"]) + oracle.kv_cache_bytes(rows, c["v_bits"]) == c["bytes"]
    assert c["bytes"] / 2 ** 30 == 0.375


# ---- cache layout -----------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_k_layout_bijection_and_locality(bits):
    pos = [oracle.kv_k_pos(bits, d) for d in range(D)]
    assert sorted(pos) == list(range(D))
    for t in range(4):
        for j in range(4):
            # lane quarter t, matrix step j: values d = 32j + 8t + s fill 8 consecutive slots
            got = sorted(pos[32 * j + 8 * t + s] for s in range(8))
            assert got == list(range(32 * t + 8 * j, 32 * t + 8 * j + 8))
    if bits == 4:
        for d in range(0, D, 2):  # a pair (s, s+1) sits four nibbles apart in one 32-bit word
            assert pos[d + 1] - pos[d] == 4 and pos[d] // 8 == pos[d + 1] // 8


@pytest.mark.parametrize("bits", [4, 8])
def test_v_layout_bijection_and_locality(bits):
    pos = {(w, d): oracle.kv_v_pos(bits, w, d) for w in range(32) for d in range(D)}
    assert sorted(pos.values()) == list(range(32 * D))
    tau = lambda t, s: 4 * t + s if s < 4 else 16 + 4 * t + (s - 4)
    P = 128 // bits  # values per 16-byte piece
    for t in range(4):
        for r in range(16):
            lane = 16 * t + r
            for c in range(8):
                # lane (t, r), slice c: its eight tokens at d = 16c + r fill 8 consecutive slots
                got = sorted(pos[(tau(t, s), 16 * c + r)] for s in range(8))
                e = c // (P // 8)
                base = 64 * P * e + P * lane + 8 * (c % (P // 8))
                assert got == list(range(base, base + 8))
    # piece e of every lane: the 64 lanes' pieces tile one contiguous 1 KB block
    for e in range(bits // 2):
        lanes = sorted(min(pos[(tau(t, s), 16 * c + r)] for s in range(8) for c in range(8)
                           if c // (P // 8) == e) for t in range(4) for r in range(16))
        assert lanes == [64 * P * e + P * l for l in range(64)]


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bits", [4, 8])
def test_layout_round_trip(which, bits):
    cap, regions = 64, 3
    rows = cap * regions
    rng = np.random.default_rng(7 + which + bits)
    codes = rng.integers(0, 1 << bits, (rows, D), dtype=np.uint8)
    slots = rng.permutation(rows).astype(np.int64)
    cache = oracle.kv_layout(codes, slots, which, bits, cap, rows)
    assert cache.nbytes == rows * D * bits // 8
    back = oracle.kv_unlayout(cache, slots, which, bits, cap)
    assert (back == codes).all()
    # a partial write leaves every other row untouched
    cache2 = oracle.kv_layout(codes[:5], slots[:5], which, bits, cap, rows, cache=cache.copy())
    assert (cache2 == cache).all()


# ---- attention --------------------------------------------------------------------------

def _cache(B, Hkv, cap, kbits, kg, vbits, vg, seed):
    rows = B * Hkv * cap
    k = _rows(rows, seed)
    v = _rows(rows, seed + 1)
    kc, ks = oracle.kv_quantize(k, kbits, kg)
    vc, vs = oracle.kv_quantize(v, vbits, vg)
    return kc, ks, vc, vs


def _reference(q, kc, ks, vc, vs, lens, Hkv, cap, kbits, vbits, sm):
    """The same attention through scipy's softmax and numpy products."""
    B, Hq, _ = q.shape
    K = _deq(kc, ks, kbits).reshape(B, Hkv, cap, D)
    V = _deq(vc, vs, vbits).reshape(B, Hkv, cap, D)
    o = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            L = lens[b]
            if L == 0:
                continue
            z = sm * (K[b, hk, :L] @ q[b, h].astype(np.float64))
            o[b, h] = softmax(z) @ V[b, hk, :L]
    return o


@pytest.mark.parametrize("kbits,vbits,kg,vg", [(4, 8, 64, 64), (8, 8, 32, 128), (4, 4, 128, 32)])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_attention_matches_library_softmax(kbits, vbits, kg, vg, Hq, Hkv):
    B, cap = 2, 64
    lens = np.array([37, 64], np.int32)
    kc, ks, vc, vs = _cache(B, Hkv, cap, kbits, kg, vbits, vg, 100 + kbits + Hq)
    q = np.random.default_rng(5).standard_normal((B, Hq, D)).astype(np.float16)
    sm = 1 / math.sqrt(D)
    o, a = oracle.attn_decode(q, kc, ks, vc, vs, lens, Hkv, cap, kbits, vbits, sm)
    ref = _reference(q, kc, ks, vc, vs, lens, Hkv, cap, kbits, vbits, sm)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)
    assert (a >= np.abs(o) - 1e-15).all()


def test_attention_single_token_returns_v():
    B, Hkv, cap = 1, 2, 32
    kc, ks, vc, vs = _cache(B, Hkv, cap, 4, 64, 8, 64, 3)
    q = _rows(4, 9).reshape(1, 4, D)
    o, a = oracle.attn_decode(q, kc, ks, vc, vs, np.array([1], np.int32), Hkv, cap, 4, 8, 0.3)
    V = _deq(vc, vs, 8).reshape(Hkv, cap, D)
    for h in range(4):
        assert (o[0, h] == V[h // 2, 0]).all()
        assert (a[0, h] == np.abs(V[h // 2, 0])).all()


def test_attention_zero_query_is_mean():
    B, Hkv, cap = 1, 1, 64
    kc, ks, vc, vs = _cache(B, Hkv, cap, 8, 32, 8, 32, 4)
    q = np.zeros((1, 2, D), np.float16)
    o, _ = oracle.attn_decode(q, kc, ks, vc, vs, np.array([50], np.int32), Hkv, cap, 8, 8, 1.0)
    V = _deq(vc, vs, 8)[:50]
    assert np.allclose(o[0, 0], V.mean(axis=0), rtol=1e-13, atol=1e-15)
    assert (o[0, 0] == o[0, 1]).all()


def test_attention_two_tokens_closed_form():
    B, Hkv, cap = 1, 1, 32
    kc, ks, vc, vs = _cache(B, Hkv, cap, 4, 128, 8, 128, 6)
    q = _rows(1, 12).reshape(1, 1, D)
    sm = 0.125
    o, _ = oracle.attn_decode(q, kc, ks, vc, vs, np.array([2], np.int32), Hkv, cap, 4, 8, sm)
    K, V = _deq(kc, ks, 4), _deq(vc, vs, 8)
    z = sm * (K[:2] @ q[0, 0].astype(np.float64))
    p1 = 1 / (1 + math.exp(z[1] - z[0]))
    assert np.allclose(o[0, 0], p1 * V[0] + (1 - p1) * V[1], rtol=1e-12, atol=1e-15)


def test_attention_token_order_and_empty():
    B, Hkv, cap = 2, 1, 32
    kc, ks, vc, vs = _cache(B, Hkv, cap, 4, 64, 8, 64, 8)
    q = _rows(2, 13).reshape(2, 1, D)
    lens = np.array([20, 0], np.int32)
    o, a = oracle.attn_decode(q, kc, ks, vc, vs, lens, Hkv, cap, 4, 8, 0.1)
    perm = np.arange(B * cap)
    perm[:20] = np.random.default_rng(1).permutation(20)
    o2, _ = oracle.attn_decode(q, kc[perm], ks[perm], vc[perm], vs[perm], lens, Hkv, cap, 4, 8, 0.1)
    assert np.allclose(o[0], o2[0], rtol=1e-13, atol=1e-15)
    assert (o[1] == 0).all() and (a[1] == 0).all()


def test_attention_length_clamped_to_capacity():
    B, Hkv, cap = 2, 1, 32
    kc, ks, vc, vs = _cache(B, Hkv, cap, 4, 64, 8, 64, 10)
    q = _rows(2, 14).reshape(2, 1, D)
    o1, _ = oracle.attn_decode(q, kc, ks, vc, vs, np.array([cap, 5], np.int32), Hkv, cap, 4, 8, 0.1)
    o2, _ = oracle.attn_decode(q, kc, ks, vc, vs, np.array([cap + 100, 5], np.int32), Hkv, cap, 4, 8, 0.1)
    assert (o1 == o2).all()
