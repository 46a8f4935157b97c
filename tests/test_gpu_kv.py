"""GPU parity of the quantized KV cache and decode attention (qkv_quantize, qattn_decode).

Write path: the cache bytes and fp32 scales after qkv_quantize equal, bit for bit, the
oracle's quantization placed by the oracle's storage map -- including rows never written
(they keep their fill pattern) and appends made over several calls.

Attention: compared element by element with the oracle's fp64 attention over the oracle's
own codes (identical to the GPU's).  Tolerance, derived from the kernel's arithmetic
(u = 2^-11, the fp16 unit roundoff): each V value is rounded to fp16 twice (its scale, then
the product: 2u), each softmax weight once (u); the weights are normalised by their fp32 sum
and o is rounded to fp16 once.  So |o - r| <= u|r| + 3u * a + (fp32 terms), where
a[d] = sum_t p_t |v_t[d]| (computed by the oracle).  The fp32 scores carry an error delta of
at most 130 * 2^-24 * sm * sum_d |q_d k_d| (natural-log units), which moves each normalised
weight by a factor within e^(+-2 delta); the test allows
    u|r| + (3.2u + 2 delta_max) * a + 1e-6 * (1 + a),
and checks that the rms error stays under 2e-3 of the rms output.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from parity import gpu, rel_err

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
FILL = 0xA5


def _dev(a, dtype=None):
    torch, _ = gpu()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class Cache:
    """A K/V cache on the device, and the oracle's copy built from the same fp16 rows."""

    def __init__(self, B, Hq, Hkv, cap, kb, vb, kg, vg, seed):
        torch, q = gpu()
        self.q = q
        self.d = q.kv_desc(B, Hq, Hkv, cap, kb, vb, kg, vg)
        self.B, self.Hq, self.Hkv, self.cap, self.kb, self.vb = B, Hq, Hkv, cap, kb, vb
        self.rows = B * Hkv * cap
        self.x = {q.QKV_K: workloads.kv_rows(self.rows, seed), q.QKV_V: workloads.kv_rows(self.rows, seed + 1)}
        self.bits = {q.QKV_K: kb, q.QKV_V: vb}
        self.g = {q.QKV_K: kg, q.QKV_V: vg}
        self.codes, self.scales = {}, {}
        for w in (q.QKV_K, q.QKV_V):
            self.codes[w] = torch.full((q.qkv_cache_bytes(self.d, w),), FILL, dtype=torch.uint8, device="cuda")
            self.scales[w] = torch.full((q.qkv_scale_count(self.d, w),), -1.0, dtype=torch.float32, device="cuda")

    def write(self, which, slots):
        """Quantize the rows at `slots` (host int64 array) through the C ABI."""
        xs = _dev(self.x[which].view(np.int16)[slots])
        sl = _dev(np.asarray(slots, np.int64))
        self.q.qkv_quantize(self.d, which, xs, 128, sl, len(slots), self.codes[which], self.scales[which])

    def write_all(self):
        for w in (self.q.QKV_K, self.q.QKV_V):
            self.write(w, np.arange(self.rows, dtype=np.int64))

    def oracle_cache(self, which, slots):
        """Oracle bytes and scales after quantizing the rows at `slots` into a FILL cache."""
        codes, scales = oracle.kv_quantize(self.x[which][slots], self.bits[which], self.g[which])
        cache = np.full(self.rows * 128 * self.bits[which] // 8, FILL, np.uint8)
        oracle.kv_layout(codes, slots, which, self.bits[which], self.cap, self.rows, cache=cache)
        sc = np.full((self.rows, 128 // self.g[which]), -1.0, np.float32)
        sc[slots] = scales
        return cache, sc.reshape(-1)

    def oracle_all(self):
        kc, ks = oracle.kv_quantize(self.x[self.q.QKV_K], self.kb, self.g[self.q.QKV_K])
        vc, vs = oracle.kv_quantize(self.x[self.q.QKV_V], self.vb, self.g[self.q.QKV_V])
        return kc, ks, vc, vs

    def attend(self, qv, lens, sm):
        torch, q = gpu()
        o = torch.empty((self.B, self.Hq, 128), dtype=torch.int16, device="cuda")
        wsb = q.qattn_decode_workspace_bytes(self.d)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        q.qattn_decode(self.d, _dev(qv.view(np.int16)), self.codes[q.QKV_K], self.scales[q.QKV_K],
                       self.codes[q.QKV_V], self.scales[q.QKV_V], _dev(np.asarray(lens, np.int32)), sm, o, ws, wsb)
        torch.cuda.synchronize()
        return o.cpu().numpy().view(np.float16).astype(np.float64)


def _score_slack(qv, kc, ks, c: Cache, lens, sm):
    """2 * delta: delta bounds the fp32 error of a score in natural-log units, 130 * 2^-24 times
    sm * max_t sum_d |q_d| |k_t[d]| (the matrix-core and scale accumulations over 128 terms);
    a score error delta changes each normalised weight by at most a factor e^(2 delta)."""
    g = 128 // ks.shape[1]
    K = np.abs((kc.astype(np.int64) - (1 << (c.kb - 1))) * np.repeat(ks.astype(np.float64), g, axis=1))
    K = K.reshape(c.B, c.Hkv, c.cap, 128)
    grp = c.Hq // c.Hkv
    worst = 0.0
    for b in range(c.B):
        L = int(lens[b])
        if L <= 0:
            continue
        for hk in range(c.Hkv):
            Q = np.abs(qv[b, hk * grp:(hk + 1) * grp].astype(np.float64))
            worst = max(worst, float((K[b, hk, :L] @ Q.T).max()))
    return 2 * 130 * 2.0 ** -24 * abs(sm) * worst


def check_attention(c: Cache, lens, sm, seed, tag=""):
    print(f"attention case {tag} lens={list(lens)[:8]}", flush=True)
    qv = workloads.kv_queries(c.B, c.Hq, seed)
    o = c.attend(qv, lens, sm)
    kc, ks, vc, vs = c.oracle_all()
    r, a = oracle.attn_decode(qv, kc, ks, vc, vs, lens, c.Hkv, c.cap, c.kb, c.vb, sm)
    slack = _score_slack(qv, kc, ks, c, lens, sm)
    bound = U * np.abs(r) + (3.2 * U + slack) * a + 1e-6 * (1.0 + a)
    err = np.abs(o - r)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (tag, worst, o[worst], r[worst], a[worst], slack, rel_err(o, r))
    # the rounding errors are independent: their rms stays far below the worst-case bound
    assert np.sqrt(np.mean(err ** 2)) <= 2e-3 * np.sqrt(np.mean(r ** 2)), (tag, rel_err(o, r))
    return o, r


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantize_bit_exact(which, bits, g):
    print(f"kv quantize which={which} bits={bits} g={g}", flush=True)
    c = Cache(2, 4, 2, 96, bits, bits, g, g, 6100 + 10 * bits + g)
    c.x[which][7, :] = 0                 # an all-zero row
    c.x[which][9, :64] = 0               # an all-zero half row
    rng = np.random.default_rng(3)
    slots = rng.permutation(c.rows)[: c.rows - 40].astype(np.int64)  # 40 rows never written
    c.write(which, slots)
    cache, sc = c.oracle_cache(which, slots)
    got = c.codes[which].cpu().numpy()
    assert np.array_equal(got, cache), np.flatnonzero(got != cache)[:10]
    assert np.array_equal(c.scales[which].cpu().numpy().view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
def test_append_over_calls(bits):
    """A prefill write followed by one-token appends per sequence equals one write of all rows."""
    c = Cache(3, 2, 2, 64, bits, bits, 64, 64, 6200 + bits)
    _, q = gpu()
    region = np.arange(c.B * c.Hkv, dtype=np.int64) * c.cap
    written = []
    for w in (q.QKV_K, q.QKV_V):
        pre = (region[:, None] + np.arange(40)[None, :]).reshape(-1)
        c.write(w, pre)
        for t in range(40, 45):
            c.write(w, region + t)
        written = np.concatenate([pre] + [region + t for t in range(40, 45)])
        cache, sc = c.oracle_cache(w, written)
        assert np.array_equal(c.codes[w].cpu().numpy(), cache)
        assert np.array_equal(c.scales[w].cpu().numpy().view(np.uint32), sc.view(np.uint32))


def test_out_of_range_slots_are_skipped():
    c = Cache(1, 2, 2, 32, 4, 8, 64, 64, 6300)
    _, q = gpu()
    slots = np.array([3, -1, c.rows, 5], np.int64)
    torch, _ = gpu()
    xs = _dev(c.x[q.QKV_V].view(np.int16)[[3, 0, 1, 5]])
    q.qkv_quantize(c.d, q.QKV_V, xs, 128, _dev(slots), 4, c.codes[q.QKV_V], c.scales[q.QKV_V])
    cache, sc = c.oracle_cache(q.QKV_V, np.array([3, 5], np.int64))
    assert np.array_equal(c.codes[q.QKV_V].cpu().numpy(), cache)
    assert np.array_equal(c.scales[q.QKV_V].cpu().numpy().view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("kb,vb,kg,vg", [(4, 8, 64, 64), (4, 4, 64, 64), (8, 8, 128, 128), (8, 4, 32, 32),
                                         (4, 8, 128, 32), (4, 8, 32, 128)])
def test_attention_formats(kb, vb, kg, vg):
    c = Cache(3, 8, 2, 256, kb, vb, kg, vg, 6400 + kb + vb + kg + vg)
    c.write_all()
    check_attention(c, np.array([256, 1, 77], np.int32), 1 / math.sqrt(128), 6401, f"{kb}{vb}{kg}{vg}")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 4), (32, 2), (5, 1), (16, 1)])
def test_attention_heads(Hq, Hkv):
    c = Cache(2, Hq, Hkv, 160, 4, 8, 64, 64, 6500 + Hq)
    c.write_all()
    check_attention(c, np.array([160, 95], np.int32), 0.0883883, 6501 + Hq, f"Hq{Hq}Hkv{Hkv}")


def test_attention_ragged_and_empty():
    lens = np.array([0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 300], np.int32)
    c = Cache(len(lens), 4, 2, 256, 4, 8, 64, 64, 6600)
    c.write_all()
    o, _ = check_attention(c, lens, 0.125, 6601, "ragged")
    assert (o[0] == 0).all()  # empty sequence


def test_attention_many_chunks():
    """One sequence and two kv heads split into many chunks merged by the second kernel."""
    c = Cache(1, 8, 2, 4096, 4, 8, 64, 64, 6700)
    _, q = gpu()
    assert q.qattn_decode_workspace_bytes(c.d) > 0
    c.write_all()
    check_attention(c, np.array([4000], np.int32), 1 / math.sqrt(128), 6701, "chunks")


def test_attention_split_rounds_down():
    """24 (sequence, kv head) rows at 1280 tokens: ten chunks of 128 each (240 workgroups)."""
    c = Cache(3, 16, 8, 1280, 4, 8, 64, 64, 6750)
    c.write_all()
    check_attention(c, np.array([1280, 700, 5], np.int32), 1 / math.sqrt(128), 6751, "split10")


def test_attention_large_scores():
    """Sharp softmax (scores of order 100): the running maximum and rescaling carry it."""
    c = Cache(2, 4, 4, 256, 8, 8, 64, 64, 6800)
    c.write_all()
    check_attention(c, np.array([256, 200], np.int32), 2.0, 6801, "sharp")


@pytest.mark.parametrize("name", ["KV_MHA", "KV_GQA"])
def test_attention_full_size(name):
    """The benchmark's shapes at full length, every output checked."""
    cfg = getattr(workloads, name)
    c = Cache(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["capacity"], 4, 8, 64, 64,
              workloads.seed_for(6))
    c.write_all()
    lens = np.full(cfg["batch"], cfg["capacity"], np.int32)
    check_attention(c, lens, 1 / math.sqrt(128), workloads.seed_for(6) + 2, name)
