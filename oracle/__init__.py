"""CPU oracle for the weight-only mixed-bit quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of
the benchmark may use this package; the product library never does.  It is a thin
ctypes wrapper over ``qoracle.c`` (plain C, fp32 quantizer as stated by the pages,
fp64 matmuls).  See the header of ``qoracle.c`` for the passages each routine follows.

Parity pins: every routine here is pinned by tests/test_oracle_*.py against the pages'
printed values, closed forms, invariants and brute force on tiny inputs, except the
device layout (``pack_device``), which is the library's own encoding: it is pinned by
round trips, by its byte map being a bijection with the documented locality, and by an
independent decoder of the documented pair rule in the tests ("parity unpinned" against
the pages, which define no device layout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "qoracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None

GROUP = 128


def build(force: bool = False) -> Path:
    """Compile qoracle.c with gcc (IEEE fp32/fp64, no contraction, OpenMP)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
            "-shared", "-fPIC", str(_SRC), "-o", str(tmp), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(str(_LIB))
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.or_half_value.restype = dbl
        L.or_half_value.argtypes = [ctypes.c_uint16]
        L.or_round_half.restype = ctypes.c_uint16
        L.or_round_half.argtypes = [dbl]
        L.or_quantize_group.restype = None
        L.or_quantize_group.argtypes = [vp, i32, i32, vp, vp, vp]
        L.or_quantize_group_sym.restype = None
        L.or_quantize_group_sym.argtypes = [vp, i32, i32, vp, vp]
        L.or_outlier_count.restype = i64
        L.or_outlier_count.argtypes = [i64, i64, dbl]
        L.or_quantize.restype = i32
        L.or_quantize.argtypes = [i64, i64, i32, i32, i32, vp, i64, dbl, vp, vp, vp, vp, vp, vp,
                                  i64, ctypes.POINTER(i64)]
        L.or_unit_values.restype = i32
        L.or_unit_values.argtypes = [i32]
        L.or_unit_bytes.restype = i32
        L.or_unit_bytes.argtypes = [i32]
        for name in ("or_pack_canonical", "or_unpack_canonical"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [i64, i64, i32, vp, vp]
        for name in ("or_pack_device", "or_unpack_device"):
            getattr(L, name).restype = i32
            getattr(L, name).argtypes = [i64, i64, i32, vp, vp]
        L.or_device_offset.restype = i64
        L.or_device_offset.argtypes = [i64, i64, i64, i32]
        L.or_device_reorder.restype = None
        L.or_device_reorder.argtypes = [i64, i64, i32, vp, vp, i32]
        L.or_linear.restype = None
        L.or_linear.argtypes = [i64, i64, i64, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp, i64]
        L.or_moe_ffn.restype = None
        L.or_moe_ffn.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp] + [vp] * 9 + [vp]
        L.or_act_quantize.restype = None
        L.or_act_quantize.argtypes = [i64, i64, vp, i64, vp, vp]
        L.or_act_pos.restype = i64
        L.or_act_pos.argtypes = [i64]
        L.or_act_layout.restype = None
        L.or_act_layout.argtypes = [i64, i64, vp, vp, i32]
        L.or_linear_a8.restype = None
        L.or_linear_a8.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
        L.or_e4m3_value.restype = dbl
        L.or_e4m3_value.argtypes = [i32]
        L.or_e4m3_ceil.restype = i32
        L.or_e4m3_ceil.argtypes = [ctypes.c_float]
        L.or_quantize_fp8.restype = i32
        L.or_quantize_fp8.argtypes = [i64, i64, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp, i32, vp]
        L.or_zero_row_bytes.restype = i64
        L.or_zero_row_bytes.argtypes = [i64, i32]
        for name in ("or_pack_zeros", "or_unpack_zeros"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [i64, i64, i32, vp, vp]
        L.or_kv_quantize_row.restype = None
        L.or_kv_quantize_row.argtypes = [vp, i32, i32, i32, vp, vp]
        L.or_kv_quantize_rows.restype = None
        L.or_kv_quantize_rows.argtypes = [vp, i64, i32, i32, vp, vp]
        L.or_kv_k_pos.restype = i64
        L.or_kv_k_pos.argtypes = [i32, i32]
        L.or_kv_v_pos.restype = i64
        L.or_kv_v_pos.argtypes = [i32, i32, i32]
        for name in ("or_kv_layout", "or_kv_unlayout"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [i32, i32, i64, i64, vp, vp, vp]
        L.or_attn_decode.restype = None
        L.or_attn_decode.argtypes = [i64, i64, i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, dbl,
                                     vp, vp]
        L.or_swiglu_act.restype = None
        L.or_swiglu_act.argtypes = [i64, i64, i32, vp] + [vp] * 6 + [vp]
        L.or_quant_bytes.restype = dbl
        L.or_quant_bytes.argtypes = [dbl] * 5
        L.or_kv_bytes.restype = dbl
        L.or_kv_bytes.argtypes = [dbl] * 5
        L.or_num_threads.restype = i32
        L.or_num_threads.argtypes = []
        L.or_set_num_threads.restype = None
        L.or_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _bits16(a):
    """fp16 array -> its uint16 bit patterns (a view, no arithmetic)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16)


# ---- fp16 -------------------------------------------------------------------------

def half_value(h: int) -> float:
    return lib().or_half_value(int(h))


def round_half(x: float) -> int:
    return lib().or_round_half(float(x))


# ---- quantizer ----------------------------------------------------------------------

def quantize_group(w_fp16, bits: int):
    """One group -> (scale_bits uint16, zero uint8, codes uint8[n])."""
    w = _bits16(w_fp16).ravel()
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint8)
    q = np.zeros(w.size, np.uint8)
    lib().or_quantize_group(_p(w), w.size, bits, _p(s), _p(z), _p(q))
    return int(s[0]), int(z[0]), q


def quantize_group_sym(w_fp16, bits: int):
    """One symmetric group -> (scale_bits uint16, codes uint8[n]); zero point 2^(bits-1)."""
    w = _bits16(w_fp16).ravel()
    s = np.zeros(1, np.uint16)
    q = np.zeros(w.size, np.uint8)
    lib().or_quantize_group_sym(_p(w), w.size, bits, _p(s), _p(q))
    return int(s[0]), q


def outlier_count(n: int, k: int, frac: float) -> int:
    return lib().or_outlier_count(n, k, frac)


def quantize(w_fp16, bits: int, outlier_frac: float = 0.0, g: int = GROUP, sym: bool = False):
    """W [N, K] fp16 -> dict(codes u8 [N,K], scales u16 [N,K/g], zeros u8 [N,K/g],
    rowptr i32 [N+1], col i32 [nnz], val u16 [nnz], sym).  With sym the groups are
    symmetric and `zeros` holds the implied midpoint 2^(bits-1) everywhere."""
    w = _bits16(w_fp16)
    N, K = w.shape
    G = K // g
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, G), np.uint16)
    zeros = np.zeros((N, G), np.uint8)
    kout = outlier_count(N, K, outlier_frac)
    rowptr = np.zeros(N + 1, np.int32)
    col = np.zeros(max(kout, 1), np.int32)
    val = np.zeros(max(kout, 1), np.uint16)
    nnz = ctypes.c_int64(0)
    rc = lib().or_quantize(N, K, bits, g, 1 if sym else 0, _p(w), K, outlier_frac, _p(codes), _p(scales),
                           None if sym else _p(zeros), _p(rowptr), _p(col), _p(val), kout, ctypes.byref(nnz))
    if rc != 0:
        raise ValueError(f"or_quantize failed rc={rc}")
    if sym:
        zeros[:] = 1 << (bits - 1)
    return dict(codes=codes, scales=scales, zeros=zeros, rowptr=rowptr,
                col=col[:nnz.value], val=val[:nnz.value], sym=sym, g=g)


# ---- packing -------------------------------------------------------------------------

def unit_values(bits: int) -> int:
    return lib().or_unit_values(bits)


def unit_bytes(bits: int) -> int:
    return lib().or_unit_bytes(bits)


def pack_canonical(codes, bits: int):
    c = _c(codes, np.uint8)
    N, K = c.shape
    out = np.zeros(N * K * bits // 8, np.uint8)
    lib().or_pack_canonical(N, K, bits, _p(c), _p(out))
    return out


def unpack_canonical(packed, N: int, K: int, bits: int):
    p = _c(packed, np.uint8)
    out = np.zeros((N, K), np.uint8)
    lib().or_unpack_canonical(N, K, bits, _p(p), _p(out))
    return out


def pack_device(codes, bits: int):
    c = _c(codes, np.uint8)
    N, K = c.shape
    out = np.zeros(N * K * bits // 8, np.uint8)
    if lib().or_pack_device(N, K, bits, _p(c), _p(out)) != 0:
        raise ValueError("device layout needs N % 16 == 0 and K % 256 == 0")
    return out


def unpack_device(packed, N: int, K: int, bits: int):
    p = _c(packed, np.uint8)
    out = np.zeros((N, K), np.uint8)
    if lib().or_unpack_device(N, K, bits, _p(p), _p(out)) != 0:
        raise ValueError("device layout needs N % 16 == 0 and K % 256 == 0")
    return out


def device_offset(n: int, cb: int, K: int, bits: int) -> int:
    return lib().or_device_offset(n, cb, K, bits)


def device_reorder(codes, bits: int, inverse: bool = False):
    """Step 1 of the device layout: codes reordered inside their packing groups."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = c.shape
    out = np.empty_like(c)
    lib().or_device_reorder(N, K, bits, _p(c), _p(out), 1 if inverse else 0)
    return out


# ---- matmuls -------------------------------------------------------------------------

def _group_of(q: dict, K: int) -> int:
    """Group size of a quantized matrix (recorded by quantize, else from the scale shape)."""
    g = q.get("g") or K // np.asarray(q["scales"]).shape[1]
    assert K % g == 0 and np.asarray(q["scales"]).shape[1] == K // g
    return g


def linear(x_fp16, q: dict, outliers: bool = True):
    """fp64 r = x * What^T (+ CSR add-back).  x [M, K] fp16; q as returned by quantize."""
    x = _bits16(x_fp16)
    M, K = x.shape
    codes = _c(q["codes"], np.uint8)
    N = codes.shape[0]
    assert codes.shape[1] == K
    g = _group_of(q, K)
    r = np.zeros((M, N), np.float64)
    use_csr = outliers and q.get("rowptr") is not None and len(q.get("col", [])) > 0
    lib().or_linear(M, N, K, g, _p(x), K, _p(codes), _p(_c(q["scales"], np.uint16)),
                    _p(_c(q["zeros"], np.uint8)),
                    _p(_c(q["rowptr"], np.int32)) if use_csr else None,
                    _p(_c(q["col"], np.int32)) if use_csr else None,
                    _p(_c(q["val"], np.uint16)) if use_csr else None, _p(r), N)
    return r


def moe_ffn(x_fp16, ids, wts, gate: list, up: list, down: list):
    """fp64 routed-expert FFN.  gate/up/down: per-expert dicts from quantize() (one group size)."""
    x = _bits16(x_fp16)
    T, D = x.shape
    ids = _c(ids, np.int32)
    wts = _c(wts, np.float32)
    topk = ids.shape[1]
    F = gate[0]["codes"].shape[0]
    g = _group_of(gate[0], D)
    assert _group_of(down[0], F) == g
    st = lambda lst, key, dt: np.ascontiguousarray(np.stack([d[key] for d in lst]), dtype=dt)
    arrs = [st(gate, "codes", np.uint8), st(gate, "scales", np.uint16), st(gate, "zeros", np.uint8),
            st(up, "codes", np.uint8), st(up, "scales", np.uint16), st(up, "zeros", np.uint8),
            st(down, "codes", np.uint8), st(down, "scales", np.uint16), st(down, "zeros", np.uint8)]
    r = np.zeros((T, D), np.float64)
    lib().or_moe_ffn(T, D, F, topk, g, _p(ids), _p(wts), _p(x), *[_p(a) for a in arrs], _p(r))
    return r


def act_quantize(x_fp16):
    """Per-token int8 activations: x [M, K] fp16 -> (xq int8 [M, K] row-major, scales fp32 [M])."""
    x = _bits16(x_fp16)
    M, K = x.shape
    xq = np.zeros((M, K), np.int8)
    sc = np.zeros(M, np.float32)
    lib().or_act_quantize(M, K, _p(x), K, _p(xq), _p(sc))
    return xq, sc


def act_pos(k: int) -> int:
    return lib().or_act_pos(k)


def act_layout(xq, inverse: bool = False):
    """Row-major int8 activations <-> the library's storage order (within 128-k groups)."""
    a = np.ascontiguousarray(xq, dtype=np.int8)
    M, K = a.shape
    out = np.zeros_like(a)
    lib().or_act_layout(M, K, _p(a), _p(out), 1 if inverse else 0)
    return out


def linear_a8(xq, sx, q: dict):
    """fp64 r = s_x * sum_g s_w * (integer group dot products of xq with q - zp)."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    M, K = xq.shape
    codes = _c(q["codes"], np.uint8)
    N = codes.shape[0]
    g = _group_of(q, K)
    r = np.zeros((M, N), np.float64)
    lib().or_linear_a8(M, N, K, g, _p(xq), _p(_c(sx, np.float32)), _p(codes), _p(_c(q["scales"], np.uint16)),
                       _p(_c(q["zeros"], np.uint8)), _p(r))
    return r


def linear_a8_fp8(xq, sx, qd) -> np.ndarray:
    """fp64 r = s_x * sum_g s_w * (integer group dot products of xq with q - zp) over a
    quantize_fp8 result (its stored fp32 scales), the definition linear_a8 computes."""
    xq = np.asarray(xq, np.int64)
    M, K = xq.shape
    g = qd["g"]
    dq = qd["codes"].astype(np.int64) - np.repeat(qd["zeros"].astype(np.int64), g, 1)
    N, G = dq.shape[0], K // g
    isum = np.einsum("mgk,ngk->mng", xq.reshape(M, G, g), dq.reshape(N, G, g))  # exact integers
    r = (isum.astype(np.float64) * qd["scales_f32"].astype(np.float64)[None]).sum(2)
    return r * np.asarray(sx, np.float64)[:, None]


def e4m3_value(code: int) -> float:
    return lib().or_e4m3_value(code)


def e4m3_ceil(t: float) -> int:
    return lib().or_e4m3_ceil(t)


def quantize_fp8(w_fp16, bits: int, g: int = GROUP, sym: bool = False, fb_stride: int = 8):
    """fp8 block scales with an fp16 fallback: W [N, K] fp16 -> dict(codes u8 [N,K], sc8 u8
    [N,K/g] scale bytes, zeros u8 [N,K/g] (midpoints when sym), scales_f32 [N,K/g] stored scale
    values, factors f32 [N], fb u16 [N, fb_stride], counts i32 [N], most, g, sym)."""
    w = _bits16(w_fp16)
    N, K = w.shape
    G = K // g
    out = dict(codes=np.zeros((N, K), np.uint8), sc8=np.zeros((N, G), np.uint8), zeros=np.zeros((N, G), np.uint8),
               scales_f32=np.zeros((N, G), np.float32), factors=np.zeros(N, np.float32),
               fb=np.zeros((N, fb_stride), np.uint16), counts=np.zeros(N, np.int32))
    out["most"] = lib().or_quantize_fp8(N, K, bits, g, 1 if sym else 0, _p(w), K, _p(out["codes"]), _p(out["sc8"]),
                                        _p(out["zeros"]), _p(out["scales_f32"]), _p(out["factors"]), _p(out["fb"]),
                                        fb_stride, _p(out["counts"]))
    out["g"], out["sym"] = g, sym
    return out


def dequant_fp8(qd) -> np.ndarray:
    """fp64 W_hat = (q - zp) * stored scale for a quantize_fp8 result."""
    g = qd["g"]
    z = np.repeat(qd["zeros"].astype(np.float64), g, 1)
    s = np.repeat(qd["scales_f32"].astype(np.float64), g, 1)
    return (qd["codes"].astype(np.float64) - z) * s


def linear_fp8(x_fp16, qd) -> np.ndarray:
    """fp64 r = x * W_hat^T over the exactly dequantized fp8-scale weights (numpy matmul)."""
    return np.asarray(x_fp16, np.float16).astype(np.float64) @ dequant_fp8(qd).T


def swiglu_act_fp8(x_rows_fp16, gate: dict, up: dict) -> np.ndarray:
    """fp64 silu(What_gate x) * (What_up x) for token rows over fp8-scale weights (quantize_fp8
    dicts), before the fp16 rounding ([MoE] s4.2 expert FFN gate/up; silu(v) = v / (1 + e^-v))."""
    gv, uv = linear_fp8(x_rows_fp16, gate), linear_fp8(x_rows_fp16, up)
    return gv / (1.0 + np.exp(-gv)) * uv


def moe_ffn_fp8(x_fp16, ids, wts, gate: list, up: list, down: list) -> np.ndarray:
    """fp64 routed-expert FFN over fp8-scale experts, the same definition as moe_ffn: per token,
    sum over its top-k experts of routing weight * What_down fp16(silu(gate) * up)
    ([MoE] s4.2: routing weights as given, not renormalised)."""
    x = np.asarray(x_fp16, np.float16)
    ids = np.asarray(ids)
    wts = np.asarray(wts, np.float32)
    T = x.shape[0]
    r = np.zeros((T, down[0]["codes"].shape[0]), np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            a = swiglu_act_fp8(x[t:t + 1], gate[e], up[e]).astype(np.float16)
            r[t] += float(wts[t, j]) * linear_fp8(a, down[e])[0]
    return r


def swiglu_act(x_row_fp16, gate: dict, up: dict):
    """fp64 silu(What_gate x) * (What_up x) for one token row, before fp16 rounding."""
    xt = _bits16(x_row_fp16).ravel()
    F, D = gate["codes"].shape
    g = _group_of(gate, D)
    v = np.zeros(F, np.float64)
    lib().or_swiglu_act(D, F, g, _p(xt), _p(_c(gate["codes"], np.uint8)), _p(_c(gate["scales"], np.uint16)),
                        _p(_c(gate["zeros"], np.uint8)), _p(_c(up["codes"], np.uint8)),
                        _p(_c(up["scales"], np.uint16)), _p(_c(up["zeros"], np.uint8)), _p(v))
    return v


# ---- zero points stored in b bits -----------------------------------------------------

def zero_row_bytes(G: int, bits: int) -> int:
    return lib().or_zero_row_bytes(G, bits)


def pack_zeros(zeros, bits: int):
    """u8 zero points [N][G] -> rows of b-bit fields (LSB-first), zero_row_bytes(G, bits) each."""
    z = _c(zeros, np.uint8)
    N, G = z.shape
    out = np.zeros((N, zero_row_bytes(G, bits)), np.uint8)
    lib().or_pack_zeros(N, G, bits, _p(z), _p(out))
    return out


def unpack_zeros(packed, N: int, G: int, bits: int):
    p = _c(packed, np.uint8)
    z = np.zeros((N, G), np.uint8)
    lib().or_unpack_zeros(N, G, bits, _p(p), _p(z))
    return z


# ---- quantized KV cache and decode attention ------------------------------------------

KV_DIM = 128


def kv_quantize(x_fp16, bits: int, g: int):
    """Rows of fp16 head vectors [n][128] -> (offset codes u8 [n][128], fp32 scales [n][128/g])."""
    x = np.ascontiguousarray(_bits16(x_fp16).reshape(-1, KV_DIM))
    n = x.shape[0]
    codes = np.zeros((n, KV_DIM), np.uint8)
    scales = np.zeros((n, KV_DIM // g), np.float32)
    lib().or_kv_quantize_rows(_p(x), n, g, bits, _p(codes), _p(scales))
    return codes, scales


def kv_k_pos(bits: int, d: int) -> int:
    return lib().or_kv_k_pos(bits, d)


def kv_v_pos(bits: int, w: int, d: int) -> int:
    return lib().or_kv_v_pos(bits, w, d)


def kv_cache_bytes(rows: int, bits: int) -> int:
    return rows * KV_DIM * bits // 8


def kv_layout(codes, slots, which: int, bits: int, cap: int, total_rows: int, cache=None):
    """Scatter offset codes [n][128] to cache rows `slots` (which: 0 = K, 1 = V layout)."""
    codes = _c(codes, np.uint8)
    slots = _c(slots, np.int64)
    if cache is None:
        cache = np.zeros(kv_cache_bytes(total_rows, bits), np.uint8)
    lib().or_kv_layout(which, bits, cap, len(slots), _p(slots), _p(codes), _p(cache))
    return cache


def kv_unlayout(cache, slots, which: int, bits: int, cap: int):
    cache = _c(cache, np.uint8)
    slots = _c(slots, np.int64)
    codes = np.zeros((len(slots), KV_DIM), np.uint8)
    lib().or_kv_unlayout(which, bits, cap, len(slots), _p(slots), _p(cache), _p(codes))
    return codes


def attn_decode(q_fp16, kc, ks, vc, vs, lens, kv_heads: int, cap: int, kbits: int, vbits: int,
                sm_scale: float):
    """fp64 decode attention over offset codes [B*Hkv*cap][128] and fp32 scales.
    Returns (o [B][Hq][128], a [B][Hq][128]) with a = sum_t p_t |v_t|."""
    q = _bits16(q_fp16)
    B, Hq = q.shape[0], q.shape[1]
    kc, vc = _c(kc, np.uint8), _c(vc, np.uint8)
    ks, vs = _c(ks, np.float32), _c(vs, np.float32)
    kg, vg = KV_DIM // ks.shape[1], KV_DIM // vs.shape[1]
    lens = _c(lens, np.int32)
    o = np.zeros((B, Hq, KV_DIM), np.float64)
    a = np.zeros((B, Hq, KV_DIM), np.float64)
    lib().or_attn_decode(B, Hq, kv_heads, cap, kbits, kg, vbits, vg, _p(np.ascontiguousarray(q)), _p(kc), _p(ks),
                         _p(vc), _p(vs), _p(lens), float(sm_scale), _p(o), _p(a))
    return o, a


# ---- byte accounting ----------------------------------------------------------------

def quant_bytes(numel, bits, g, scale_bytes, zp_bits) -> float:
    return lib().or_quant_bytes(float(numel), float(bits), float(g), float(scale_bytes),
                                float(zp_bits))


def kv_bytes(layers, kv_heads, head_dim, tokens, bytes_per_elem) -> float:
    return lib().or_kv_bytes(float(layers), float(kv_heads), float(head_dim), float(tokens),
                             float(bytes_per_elem))


def num_threads() -> int:
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(int(n))
