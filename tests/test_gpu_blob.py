"""A weight quantized and packed on the GPU, serialized to a blob on the host, parsed and
uploaded again, gives bit-identical GEMV and GEMM outputs (outliers included)."""
import numpy as np
import pytest

import workloads
from parity import GpuWeight, from_dev_fp16, gpu, to_dev_fp16

pytestmark = pytest.mark.gpu


def test_blob_round_trip_through_device():
    torch, q = gpu()
    n, k, m, frac = 256, 1024, 20, 0.002
    w = workloads.weights_fp16(n, k, 91)
    workloads.plant_outliers(w, frac, 91)
    g = GpuWeight(w, 5, frac)
    host = dict(packed=g.packed.cpu().numpy(), scales=g.scales.cpu().numpy().view(np.uint16),
                zeros=g.zeros.cpu().numpy(), rowptr=g.rowptr.cpu().numpy(),
                col=g.col.cpu().numpy()[: g.nnz].copy(), val=g.val.cpu().numpy().view(np.uint16)[: g.nnz].copy())
    hw = q.qp_weight(host["packed"].ctypes.data, host["scales"].ctypes.data, host["zeros"].ctypes.data,
                     host["rowptr"].ctypes.data, host["col"].ctypes.data, host["val"].ctypes.data, g.nnz)
    blob = np.zeros(q.qp_blob_bytes(g.desc, g.nnz), np.uint8)
    q.qp_blob_write(g.desc, hw, blob)
    _, d2, nnz, offs = q.qp_blob_parse(blob)
    raw = blob.tobytes()
    G = k // 128
    sec = lambda i, dt, cnt: torch.from_numpy(np.frombuffer(raw, dt, cnt, offs[i]).copy()).cuda()
    packed = sec(0, np.uint8, q.qp_packed_bytes(d2))
    scales = sec(1, np.int16, n * G)
    zeros = sec(2, np.uint8, n * G)
    rowptr, col, val = sec(3, np.int32, n + 1), sec(4, np.int32, nnz), sec(5, np.int16, nnz)
    h2 = q.weight(packed, scales, zeros, rowptr, col, val, nnz)
    x = workloads.activations_fp16(m, k, 92)
    xd = to_dev_fp16(x)
    for entry in ("qlinear_gemv", "qlinear_gemm"):
        mm = 8 if entry == "qlinear_gemv" else m
        ys = []
        for h in (g.handle(), h2):
            y = torch.empty((mm, n), dtype=torch.int16, device="cuda")
            if entry == "qlinear_gemm":
                wsb = q.qlinear_gemm_workspace_bytes(d2, mm, nnz)
                ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
                q.qlinear_gemm(d2, h, xd, k, mm, y, n, ws, wsb)
            else:
                q.qlinear_gemv(d2, h, xd, k, mm, y, n)
            torch.cuda.synchronize()
            ys.append(from_dev_fp16(y))
        assert np.array_equal(ys[0].view(np.uint16), ys[1].view(np.uint16)), entry
