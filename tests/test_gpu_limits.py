"""GPU parity at the size limits: a 6-bit weight of 43,680 x 65,536 (2,146,959,360 packed bytes,
just under 2 GiB, the largest a GEMM accepts; 2.86e9 codes, so every 32-bit element index
would wrap) through the quantizer, the packer, the decode GEMV (M = 1 and 16) and the prefill
GEMM (M = 64), checked on sampled rows against the oracle's quantization of those rows; and
grouped calls over zero routed rows.  The weights come from torch's seeded CUDA generator
(N(0, 0.02)); the sampled rows are copied to the host as input data for the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from parity import TOL, from_dev_fp16, gpu, rel_err, report, to_dev_fp16

pytestmark = pytest.mark.gpu

N, K, BITS = 43680, 65536, 6
ROWS = (0, 1, 15, 16, 17, 255, 256, 21839, 21840, 43663, 43664, 43679)


@pytest.fixture(scope="module")
def big():
    torch, q = gpu()
    dev = torch.device("cuda")
    d = q.desc(BITS, N, K, q.QP_LAYOUT_DEVICE)
    assert q.qp_packed_bytes(d) == N * K * BITS // 8 < 1 << 31
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    w = (torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.float16)
    rows = np.array(ROWS)
    w_rows = w[torch.from_numpy(rows).to(dev)].cpu().numpy()  # oracle input: the sampled rows
    G = K // 128
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, G), dtype=torch.int16, device=dev)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    dummy = torch.empty(1, dtype=torch.int32, device=dev)
    wsb = q.qpack_quantize_workspace_bytes(d, 0.0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _, nnz = q.qpack_quantize(d, w.view(torch.int16), K, 0.0, codes, scales, zeros, rp, dummy,
                              dummy.view(torch.int16), 0, ws, wsb)
    assert nnz == 0
    del w, ws
    packed = torch.empty(q.qp_packed_bytes(d), dtype=torch.uint8, device=dev)
    q.qpack_pack(d, codes, packed)
    torch.cuda.synchronize()
    got_codes = codes[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del codes
    ref = oracle.quantize(w_rows, BITS)
    yield dict(d=d, h=q.weight(packed, scales, zeros), keep=(packed, scales, zeros), rows=rows, ref=ref,
               got_codes=got_codes)
    del packed, scales, zeros
    torch.cuda.empty_cache()


def test_quantize_and_pack_at_the_largest_weight(big):
    """The sampled rows' codes equal the oracle's (the far end of a 2.86e9-code buffer)."""
    assert np.array_equal(big["got_codes"], big["ref"]["codes"])


@pytest.mark.parametrize("m", (1, 16))
def test_gemv_at_the_largest_weight(big, m):
    torch, q = gpu()
    print(f"gemv {N}x{K} {BITS}-bit m={m}", flush=True)
    x = workloads.activations_fp16(m, K, 4243 + m)
    y = torch.empty((m, N), dtype=torch.int16, device="cuda")
    q.qlinear_gemv(big["d"], big["h"], to_dev_fp16(x), K, m, y, N)
    torch.cuda.synchronize()
    got = from_dev_fp16(y)[:, big["rows"]]
    r = oracle.linear(x, big["ref"])
    assert rel_err(got, r) <= TOL, report(got, r)


def test_gemm_at_the_largest_weight(big):
    torch, q = gpu()
    m = 64
    print(f"gemm {N}x{K} {BITS}-bit m={m}", flush=True)
    x = workloads.activations_fp16(m, K, 4250)
    y = torch.empty((m, N), dtype=torch.int16, device="cuda")
    q.qlinear_gemm(big["d"], big["h"], to_dev_fp16(x), K, m, y, N, None, 0)
    torch.cuda.synchronize()
    got = from_dev_fp16(y)[:, big["rows"]]
    r = oracle.linear(x, big["ref"])
    assert rel_err(got, r) <= TOL, report(got, r)


@pytest.mark.parametrize("epi", ("none", "rows_f32"))
def test_grouped_over_zero_rows_leaves_the_output(epi):
    """rows = 0 (every expert empty): the call succeeds and writes nothing."""
    torch, q = gpu()
    n, k, E = 256, 512, 3
    from parity import GpuWeight
    ws = [GpuWeight(workloads.weights_fp16(n, k, 4260 + e), 4) for e in range(E)]
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    x = to_dev_fp16(workloads.activations_fp16(1, k, 4270))
    if epi == "none":
        y = torch.full((1, n), 0x3C00, dtype=torch.int16, device="cuda")
        q.qlinear_grouped_gemm(ws[0].desc, [w.handle() for w in ws], x, k, None, offsets, 0, q.QP_EPI_NONE, y, n)
    else:
        y = torch.full((1, n), 7.0, dtype=torch.float32, device="cuda")
        q.qlinear_grouped_gemm(ws[0].desc, [w.handle() for w in ws], x, k, None, offsets, 0, q.QP_EPI_ROWS_F32, y, n)
    torch.cuda.synchronize()
    before = 0x3C00 if epi == "none" else 7.0
    assert (y.cpu().numpy() == before).all()
