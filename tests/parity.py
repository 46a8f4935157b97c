"""Shared helpers for the parity tests (test infrastructure).

Tolerance for matmul outputs (the stated target: max relative error 2e-3 against an fp64
accumulation of the dequantized weights).  Near-zero outputs make a pure elementwise ratio
meaningless, so the denominator is floored at 1% of the output's RMS:
    err = max |y - r| / max(|r|, 0.01 * rms(r)).
The arithmetic behind 2e-3: the fp16 rounding of y alone contributes up to 2^-11 = 4.9e-4
relative; fp32 accumulation over k <= 14336 products and per-group scaling add well under
1e-5 of rms(r) (worst case about 2.6e-5 of the floor), leaving a >3x margin.
"""
from __future__ import annotations

import numpy as np

TOL = 2e-3


def rel_err(y, r) -> float:
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), 0.01 * rms)
    return float(np.max(np.abs(y - r) / den))


def report(y, r) -> str:
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    ad = np.abs(y - r)
    return (f"floored_rel={rel_err(y, r):.3e} max_abs={ad.max():.3e} rms_ref={np.sqrt(np.mean(r * r)):.3e} "
            f"unfloored_max_rel={np.max(ad / np.maximum(np.abs(r), 1e-30)):.3e}")


def fp16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16)


def gpu():
    """torch plus the binding, imported lazily so CPU-only collection never needs a GPU."""
    import torch

    import weight_only_mixed_amd as q
    return torch, q


class GpuWeight:
    """Quantized + packed weight on the device, built through the C ABI."""

    def __init__(self, w_fp16: np.ndarray, bits: int, outlier_frac: float = 0.0, layout: int = 1,
                 sym: bool = False, g: int = 128, packed_zeros: bool = False):
        """packed_zeros: affine zero points kept in b bits (QP_ZERO_PACKED, packed on the GPU
        from qpack_quantize's bytes by qpack_pack_zeros); the bytes stay in zeros_u8."""
        torch, q = gpu()
        n, k = w_fp16.shape
        dev = torch.device("cuda")
        self.n, self.k, self.bits, self.sym, self.g = n, k, bits, sym, g
        w = torch.from_numpy(np.ascontiguousarray(w_fp16).view(np.int16)).to(dev)
        mode = q.QP_ZERO_MIDPOINT if sym else (q.QP_ZERO_PACKED if packed_zeros else q.QP_ZERO_STORED)
        d = q.desc(bits, n, k, layout, group_size=g, zero_mode=mode)
        self.desc = d
        G = k // g
        self.codes = torch.empty((n, k), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((n, G), dtype=torch.int16, device=dev)
        self.zeros = torch.empty((n, G), dtype=torch.uint8, device=dev)
        kout = q.qp_outlier_count(n, k, outlier_frac)
        self.rowptr = torch.zeros(n + 1, dtype=torch.int32, device=dev)
        self.col = torch.empty(max(kout, 1), dtype=torch.int32, device=dev)
        self.val = torch.empty(max(kout, 1), dtype=torch.int16, device=dev)
        wsb = q.qpack_quantize_workspace_bytes(d, outlier_frac)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if sym:  # no zero points are written or read: pass none
            self.zeros = None
        _, self.nnz = q.qpack_quantize(d, w, k, outlier_frac, self.codes, self.scales, self.zeros,
                                       self.rowptr, self.col, self.val, kout, ws, wsb)
        del w, ws
        self.packed = torch.empty(q.qp_packed_bytes(d), dtype=torch.uint8, device=dev)
        q.qpack_pack(d, self.codes, self.packed)
        if packed_zeros:
            self.zeros_u8 = self.zeros
            self.zeros = torch.full((q.qp_zero_bytes(d),), 0xA5, dtype=torch.uint8, device=dev)
            q.qpack_pack_zeros(d, self.zeros_u8, self.zeros)

    def handle(self, with_csr: bool = True):
        _, q = gpu()
        if with_csr and self.nnz > 0:
            return q.weight(self.packed, self.scales, self.zeros, self.rowptr, self.col, self.val, self.nnz)
        return q.weight(self.packed, self.scales, self.zeros)

    def host(self) -> dict:
        """Device results copied back (for comparison with the oracle's own results)."""
        zeros = (np.full((self.n, self.k // self.g), 1 << (self.bits - 1), np.uint8) if self.sym
                 else self.zeros.cpu().numpy())
        return dict(codes=self.codes.cpu().numpy(), scales=self.scales.cpu().numpy().view(np.uint16),
                    zeros=zeros, rowptr=self.rowptr.cpu().numpy(),
                    col=self.col.cpu().numpy()[: self.nnz], val=self.val.cpu().numpy().view(np.uint16)[: self.nnz])


def to_dev_fp16(a: np.ndarray):
    torch, _ = gpu()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def from_dev_fp16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.float16)
