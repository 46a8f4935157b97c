"""Python binding of libqpack (include/qpack.h): MI355X weight-only mixed-bit linear layers.

Argument marshalling only: every function here forwards to the C entry point of the same
name, passing device pointers (torch tensors or raw integer addresses) and the current HIP
stream.  All computation runs in the library's HIP kernels; there is no fallback.  Importing
this package fails loudly if libqpack.so has not been built (``python
weight_only_mixed_amd/build.py`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
from pathlib import Path

# torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7) as the system
# one libqpack.so is linked against.  Loading torch first makes libqpack bind to the
# runtime torch already initialised, so both share one runtime (and one view of devices,
# streams and memory) in the process.
import torch  # noqa: F401  (import order matters, see above)

_LIB_PATH = Path(__file__).resolve().parent / "libqpack.so"
if not _LIB_PATH.exists():
    raise ImportError(f"{_LIB_PATH} is missing: build the HIP library first "
                      "(python weight_only_mixed_amd/build.py)")
lib = ctypes.CDLL(str(_LIB_PATH))

QP_OK, QP_ERR_INVALID_ARG, QP_ERR_UNSUPPORTED, QP_ERR_DEVICE, QP_ERR_WORKSPACE = range(5)
QP_LAYOUT_CANONICAL, QP_LAYOUT_DEVICE = 0, 1
QP_EPI_NONE, QP_EPI_SWIGLU, QP_EPI_ROWS_F32 = 0, 1, 2
QP_ZERO_STORED, QP_ZERO_MIDPOINT, QP_ZERO_PACKED = 0, 1, 2
QP_SCALE_FP16, QP_SCALE_FP8 = 0, 1
STATUS_NAMES = {0: "QP_OK", 1: "QP_ERR_INVALID_ARG", 2: "QP_ERR_UNSUPPORTED", 3: "QP_ERR_DEVICE",
                4: "QP_ERR_WORKSPACE"}


class qp_weight_desc(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("zero_mode", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("scale_format", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class qp_weight(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("csr_rowptr", ctypes.c_void_p), ("csr_col", ctypes.c_void_p),
                ("csr_val", ctypes.c_void_p), ("nnz", ctypes.c_int64),
                ("scales8", ctypes.c_void_p), ("row_factors", ctypes.c_void_p), ("fb_scales", ctypes.c_void_p),
                ("fb_stride", ctypes.c_int64)]


class qkv_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("k_group", ctypes.c_int32), ("v_group", ctypes.c_int32), ("capacity", ctypes.c_int64)]


QKV_K, QKV_V = 0, 1


class qp_gemv_problem(ctypes.Structure):
    _fields_ = [("desc", qp_weight_desc), ("w", qp_weight), ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
                ("m", ctypes.c_int64), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


_vp, _i64, _i32, _dbl, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
_D = ctypes.POINTER(qp_weight_desc)
_W = ctypes.POINTER(qp_weight)
_KD = ctypes.POINTER(qkv_desc)
_SIGS = {
    "qp_packed_bytes": (_sz, [_D]),
    "qp_num_groups": (_sz, [_D]),
    "qp_zero_bytes": (_sz, [_D]),
    "qp_quant_bytes": (_dbl, [_dbl] * 5),
    "qp_outlier_count": (_i64, [_i64, _i64, _dbl]),
    "qpack_quantize_workspace_bytes": (_sz, [_D, _dbl]),
    "qpack_quantize": (_i32, [_D, _vp, _i64, _dbl, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                              ctypes.POINTER(_i64), _vp, _sz, _vp]),
    "qpack_quantize_fp8": (_i32, [_D, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "qpack_pack": (_i32, [_D, _vp, _vp, _vp]),
    "qpack_unpack": (_i32, [_D, _vp, _vp, _vp]),
    "qpack_pack_zeros": (_i32, [_D, _vp, _vp, _vp]),
    "qlinear_gemv": (_i32, [_D, _W, _vp, _i64, _i64, _vp, _i64, _vp]),
    "qlinear_gemv_batch": (_i32, [ctypes.POINTER(qp_gemv_problem), _i32, _vp]),
    "qlinear_gemm_workspace_bytes": (_sz, [_D, _i64, _i64]),
    "qlinear_gemm": (_i32, [_D, _W, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp]),
    "qact_quantize": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "qlinear_gemm_a8": (_i32, [_D, _W, _vp, _vp, _i64, _vp, _i64, _vp]),
    "qlinear_grouped_gemm": (_i32, [_D, _W, _i32, _vp, _i64, _vp, _vp, _i64, _i32, _vp, _i64, _vp]),
    "qmoe_dispatch": (_i32, [_vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "qmoe_combine": (_i32, [_vp, _i64, _vp, _vp, _i64, _i32, _i64, _vp, _i64, _vp]),
    "qmoe_ffn_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64]),
    "qmoe_ffn": (_i32, [_D, _W, _D, _W, _i32, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _i64, _vp, _sz,
                        _vp]),
    "qkv_cache_bytes": (_sz, [_KD, _i32]),
    "qkv_scale_count": (_sz, [_KD, _i32]),
    "qkv_quantize": (_i32, [_KD, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "qattn_decode_workspace_bytes": (_sz, [_KD]),
    "qattn_decode": (_i32, [_KD, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _sz, _vp]),
    "qattn_decode_noalloc": (_i32, [_KD, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "qlinear_gemv_host": (_i32, [_D, _W, _vp, _i64, _i64, _vp, _i64, _i32]),
    "qlinear_gemv_host_isa": (ctypes.c_char_p, []),
    "qp_blob_bytes": (_sz, [_D, _i64]),
    "qp_blob_write": (_i32, [_D, _W, _vp, _sz]),
    "qp_blob_parse": (_i32, [_vp, _sz, _D, ctypes.POINTER(_i64), ctypes.POINTER(_sz)]),
    "qp_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class QPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {last_error()}")


def last_error() -> str:
    return lib.qp_last_error().decode()


def _ptr(t):
    """Device address of a torch tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status, check):
    if check and status != QP_OK:
        raise QPError(fn, status)
    return status


def desc(bits: int, n: int, k: int, layout: int = QP_LAYOUT_DEVICE, group_size: int = 128,
         zero_mode: int = QP_ZERO_STORED, scale_format: int = QP_SCALE_FP16):
    return qp_weight_desc(bits, group_size, layout, zero_mode, n, k, scale_format, 0)


def weight(packed, scales, zeros, rowptr=None, col=None, val=None, nnz: int = 0):
    return qp_weight(_ptr(packed), _ptr(scales), _ptr(zeros), _ptr(rowptr), _ptr(col), _ptr(val), nnz)


def weight_fp8(packed, scales8, row_factors, fb_scales, fb_stride: int, zeros=None):
    """A QP_SCALE_FP8 weight (no outliers): scale bytes, row factors, fallback list."""
    return qp_weight(_ptr(packed), None, _ptr(zeros), None, None, None, 0, _ptr(scales8), _ptr(row_factors),
                     _ptr(fb_scales), fb_stride)


# ---- host accounting ----------------------------------------------------------------

def qp_packed_bytes(d) -> int:
    return lib.qp_packed_bytes(ctypes.byref(d))


def qp_num_groups(d) -> int:
    return lib.qp_num_groups(ctypes.byref(d))


def qp_zero_bytes(d) -> int:
    return lib.qp_zero_bytes(ctypes.byref(d))


def qp_quant_bytes(numel, bits, group, scale_bytes, zp_bits) -> float:
    return lib.qp_quant_bytes(float(numel), float(bits), float(group), float(scale_bytes), float(zp_bits))


def qp_outlier_count(n: int, k: int, frac: float) -> int:
    return lib.qp_outlier_count(n, k, frac)


def qpack_quantize_workspace_bytes(d, outlier_frac: float) -> int:
    return lib.qpack_quantize_workspace_bytes(ctypes.byref(d), outlier_frac)


def qmoe_ffn_workspace_bytes(tokens, topk, n_experts, d_model, d_ff) -> int:
    return lib.qmoe_ffn_workspace_bytes(tokens, topk, n_experts, d_model, d_ff)


# ---- device entry points -----------------------------------------------------------

def qpack_quantize(d, w, ldw, outlier_frac, codes, scales, zeros, csr_rowptr=None, csr_col=None,
                   csr_val=None, csr_cap=0, workspace=None, ws_bytes=0, stream=None, check=True):
    """Returns (status, nnz)."""
    nnz = _i64(0)
    st = lib.qpack_quantize(ctypes.byref(d), _ptr(w), ldw, outlier_frac, _ptr(codes), _ptr(scales),
                            _ptr(zeros), _ptr(csr_rowptr), _ptr(csr_col), _ptr(csr_val), csr_cap,
                            ctypes.byref(nnz), _ptr(workspace), ws_bytes, _stream(stream))
    _check("qpack_quantize", st, check)
    return st, nnz.value


def qpack_quantize_fp8(d, w, ldw, codes, scales8, zeros, row_factors, fb_scales, fb_stride, counts, stream=None,
                       check=True):
    st = lib.qpack_quantize_fp8(ctypes.byref(d), _ptr(w), ldw, _ptr(codes), _ptr(scales8), _ptr(zeros),
                                _ptr(row_factors), _ptr(fb_scales), fb_stride, _ptr(counts), _stream(stream))
    return _check("qpack_quantize_fp8", st, check)


def qpack_pack(d, codes, packed, stream=None, check=True):
    return _check("qpack_pack", lib.qpack_pack(ctypes.byref(d), _ptr(codes), _ptr(packed), _stream(stream)), check)


def qpack_pack_zeros(d, zeros, packed_zeros, stream=None, check=True):
    return _check("qpack_pack_zeros", lib.qpack_pack_zeros(ctypes.byref(d), _ptr(zeros), _ptr(packed_zeros),
                                                            _stream(stream)), check)


def qpack_unpack(d, packed, codes, stream=None, check=True):
    return _check("qpack_unpack", lib.qpack_unpack(ctypes.byref(d), _ptr(packed), _ptr(codes), _stream(stream)),
                  check)


def qlinear_gemv(d, w, x, ldx, m, y, ldy, stream=None, check=True):
    return _check("qlinear_gemv", lib.qlinear_gemv(ctypes.byref(d), ctypes.byref(w), _ptr(x), ldx, m, _ptr(y),
                                                    ldy, _stream(stream)), check)


def gemv_problem(d, w, x, ldx, m, y, ldy):
    """One entry of qlinear_gemv_batch (device pointers as tensors or ints)."""
    return qp_gemv_problem(d, w, _ptr(x), ldx, m, _ptr(y), ldy)


def qlinear_gemv_batch(problems, stream=None, check=True):
    arr = (qp_gemv_problem * len(problems))(*problems)
    return _check("qlinear_gemv_batch", lib.qlinear_gemv_batch(arr, len(problems), _stream(stream)), check)


def qlinear_gemm_workspace_bytes(d, m: int, nnz: int) -> int:
    return lib.qlinear_gemm_workspace_bytes(ctypes.byref(d), m, nnz)


def qlinear_gemm(d, w, x, ldx, m, y, ldy, workspace=None, ws_bytes=0, stream=None, check=True):
    return _check("qlinear_gemm", lib.qlinear_gemm(ctypes.byref(d), ctypes.byref(w), _ptr(x), ldx, m, _ptr(y),
                                                    ldy, _ptr(workspace), ws_bytes, _stream(stream)), check)


def qact_quantize(x, ldx, m, k, xq, x_scales, stream=None, check=True):
    return _check("qact_quantize", lib.qact_quantize(_ptr(x), ldx, m, k, _ptr(xq), _ptr(x_scales), _stream(stream)),
                  check)


def qlinear_gemm_a8(d, w, xq, x_scales, m, y, ldy, stream=None, check=True):
    return _check("qlinear_gemm_a8", lib.qlinear_gemm_a8(ctypes.byref(d), ctypes.byref(w), _ptr(xq), _ptr(x_scales),
                                                          m, _ptr(y), ldy, _stream(stream)), check)


def qlinear_grouped_gemm(d, experts, x, ldx, row_src, expert_offsets, rows, epilogue, y, ldy, stream=None,
                         check=True):
    arr = (qp_weight * len(experts))(*experts)
    return _check("qlinear_grouped_gemm",
                  lib.qlinear_grouped_gemm(ctypes.byref(d), arr, len(experts), _ptr(x), ldx, _ptr(row_src),
                                           _ptr(expert_offsets), rows, epilogue, _ptr(y), ldy, _stream(stream)),
                  check)


def qmoe_dispatch(topk_ids, topk_w, tokens, topk, n_experts, expert_offsets, row_src, row_weight, token_rows,
                  stream=None, check=True):
    return _check("qmoe_dispatch",
                  lib.qmoe_dispatch(_ptr(topk_ids), _ptr(topk_w), tokens, topk, n_experts, _ptr(expert_offsets),
                                    _ptr(row_src), _ptr(row_weight), _ptr(token_rows), _stream(stream)), check)


def qmoe_combine(rows_f32, ld_rows, token_rows, row_weight, tokens, topk, n, out, ldo, stream=None, check=True):
    return _check("qmoe_combine",
                  lib.qmoe_combine(_ptr(rows_f32), ld_rows, _ptr(token_rows), _ptr(row_weight), tokens, topk, n,
                                   _ptr(out), ldo, _stream(stream)), check)


def qmoe_ffn(d_gu, gate_up, d_down, down, x, ldx, tokens, topk_ids, topk_w, topk, out, ldo, workspace, ws_bytes,
             stream=None, check=True):
    gu = (qp_weight * len(gate_up))(*gate_up)
    dn = (qp_weight * len(down))(*down)
    return _check("qmoe_ffn",
                  lib.qmoe_ffn(ctypes.byref(d_gu), gu, ctypes.byref(d_down), dn, len(gate_up), _ptr(x), ldx, tokens,
                               _ptr(topk_ids), _ptr(topk_w), topk, _ptr(out), ldo, _ptr(workspace), ws_bytes,
                               _stream(stream)), check)


# ---- quantized KV cache and decode attention --------------------------------------------

def kv_desc(batch: int, q_heads: int, kv_heads: int, capacity: int, k_bits: int = 4, v_bits: int = 8,
            k_group: int = 64, v_group: int = 64, head_dim: int = 128):
    return qkv_desc(batch, q_heads, kv_heads, head_dim, k_bits, v_bits, k_group, v_group, capacity)


def qkv_cache_bytes(d, which: int) -> int:
    return lib.qkv_cache_bytes(ctypes.byref(d), which)


def qkv_scale_count(d, which: int) -> int:
    return lib.qkv_scale_count(ctypes.byref(d), which)


def qattn_decode_workspace_bytes(d) -> int:
    return lib.qattn_decode_workspace_bytes(ctypes.byref(d))


def qkv_quantize(d, which, x, ldx, slots, rows, codes, scales, stream=None, check=True):
    return _check("qkv_quantize", lib.qkv_quantize(ctypes.byref(d), which, _ptr(x), ldx, _ptr(slots), rows,
                                                    _ptr(codes), _ptr(scales), _stream(stream)), check)


def qattn_decode(d, q, k_codes, k_scales, v_codes, v_scales, seq_lens, sm_scale, o, workspace=None, ws_bytes=0,
                 stream=None, check=True):
    return _check("qattn_decode",
                  lib.qattn_decode(ctypes.byref(d), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                   _ptr(v_scales), _ptr(seq_lens), float(sm_scale), _ptr(o), _ptr(workspace),
                                   ws_bytes, _stream(stream)), check)


def qlinear_gemv_host(d, w, x, ldx, m, y, ldy, threads: int = 0, check=True):
    """Host GEMV: w a qp_weight of HOST addresses; x, y host buffers (numpy fp16 / uint16 arrays or
    integer addresses)."""
    addr = lambda a: a if isinstance(a, int) else a.ctypes.data
    return _check("qlinear_gemv_host", lib.qlinear_gemv_host(ctypes.byref(d), ctypes.byref(w), addr(x), ldx, m,
                                                             addr(y), ldy, threads), check)


def qlinear_gemv_host_isa() -> str:
    """The vector path qlinear_gemv_host takes on this host: "avx512vbmi", "avx2" or "portable"."""
    return lib.qlinear_gemv_host_isa().decode()


def qp_blob_bytes(d, nnz: int = 0) -> int:
    return lib.qp_blob_bytes(ctypes.byref(d), nnz)


def qp_blob_write(d, w, blob, check=True):
    """w: a qp_weight of HOST addresses; blob: a writable host buffer (e.g. a numpy uint8 array)."""
    import numpy as np
    b = np.ascontiguousarray(blob)
    return _check("qp_blob_write", lib.qp_blob_write(ctypes.byref(d), ctypes.byref(w), b.ctypes.data, b.nbytes),
                  check)


def qp_blob_parse(blob, check=True):
    """-> (status, desc, nnz, section offsets (6))."""
    import numpy as np
    b = np.ascontiguousarray(blob)
    d = qp_weight_desc()
    nnz = _i64(0)
    offs = (_sz * 6)()
    st = _check("qp_blob_parse", lib.qp_blob_parse(b.ctypes.data, b.nbytes, ctypes.byref(d), ctypes.byref(nnz), offs),
                check)
    return st, d, nnz.value, list(offs)


QATTN_NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024


def qattn_decode_noalloc(d, q, k_codes, k_scales, v_codes, v_scales, seq_lens, sm_scale, o, stream=None,
                         check=True):
    return _check("qattn_decode_noalloc",
                  lib.qattn_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                           _ptr(v_scales), _ptr(seq_lens), float(sm_scale), _ptr(o),
                                           _stream(stream)), check)


EXPORTED = tuple(_SIGS)
