"""qattn_decode_noalloc (decode attention for callers that cannot allocate device memory)
against qattn_decode with a caller workspace: two calls in a row, the second on a smaller
cache, each compared bit for bit with qattn_decode on the same inputs and element by element
with the oracle's fp64 attention within the attention tolerance of the quantized-KV tests.
The second call finds the first call's partials in the shared scratch, so it also shows that
nothing stale is read."""
import numpy as np
import pytest

import oracle
import workloads
from parity import gpu
from test_gpu_kv import U, Cache, _dev, _score_slack

pytestmark = pytest.mark.gpu


def _pair(c: Cache, lens, sm, seed, tag):
    torch, q = gpu()
    print(f"noalloc case {tag}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} cap={c.cap} lens={list(lens)}", flush=True)
    qv = workloads.kv_queries(c.B, c.Hq, seed)
    qd, ln = _dev(qv.view(np.int16)), _dev(np.asarray(lens, np.int32))
    wsb = q.qattn_decode_workspace_bytes(c.d)
    assert 0 < wsb <= q.QATTN_NOALLOC_SCRATCH_BYTES, wsb
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    o_ws = torch.empty((c.B, c.Hq, 128), dtype=torch.int16, device="cuda")
    o_na = torch.full((c.B, c.Hq, 128), -1, dtype=torch.int16, device="cuda")
    K, V = q.QKV_K, q.QKV_V
    q.qattn_decode(c.d, qd, c.codes[K], c.scales[K], c.codes[V], c.scales[V], ln, sm, o_ws, ws, wsb)
    q.qattn_decode_noalloc(c.d, qd, c.codes[K], c.scales[K], c.codes[V], c.scales[V], ln, sm, o_na)
    torch.cuda.synchronize()
    a_ws, a_na = o_ws.cpu().numpy(), o_na.cpu().numpy()
    assert np.array_equal(a_na, a_ws), tag
    o = a_na.view(np.float16).astype(np.float64)
    kc, ks, vc, vs = c.oracle_all()
    r, a = oracle.attn_decode(qv, kc, ks, vc, vs, lens, c.Hkv, c.cap, c.kb, c.vb, sm)
    bound = U * np.abs(r) + (3.2 * U + _score_slack(qv, kc, ks, c, lens, sm)) * a + 1e-6 * (1.0 + a)
    assert (np.abs(o - r) <= bound).all(), tag


def test_noalloc_two_calls_second_smaller():
    sm = 1.0 / np.sqrt(128.0)
    big = Cache(2, 32, 4, 4096, 4, 8, 64, 64, 8100)      # 32 chunks per (sequence, kv head): 1.06 MB of partials
    big.write_all()
    _pair(big, [4096, 3001], sm, 8101, "first")
    small = Cache(1, 8, 2, 1024, 4, 4, 64, 64, 8200)     # 8 chunks: 33 KB of partials
    small.write_all()
    _pair(small, [777], sm, 8201, "second (smaller)")
