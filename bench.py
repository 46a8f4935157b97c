"""Benchmark: weight-only mixed-bit quantized linear layers on one MI355X.

Headline step: the 4096 x 4096 layer at 4 bits (asymmetric, groups of 128 along K, page packing
units, device tile layout) times one fp16 activation row (M = 1): one qlinear_gemv call.
Weights are quantized and packed once (the offline repack of the 70B page, s3) and the steps
rotate over enough identical copies (>= 1 GiB in total) that every weight byte is read from
HBM, as in a decode pass over distinct layers, not from the 256 MB Infinity Cache.  The timed
steps run as captured HIP graphs of back-to-back launches on one stream.

value = packed-weight bytes (codes + fp16 scales + u8 zero points) per step / step time.  The
step is one launch of the GEMV, so the roofline object (bound: HBM) is that kernel's average
launch duration over the timed region.  roofline_prefill (bound: MFMA) is the prefill
dequant-GEMM (M=512, K=8192, N=28672, 4-bit + 0.1% fp16 CSR outliers), end to end and with the
dense kernel alone.  Further lines: the 2/3/5/6-bit sweep at M = 1, 4, 8, symmetric groups,
groups of 32 and 64, zero points in b bits, a Llama-7B-shaped decode stack, a 16-expert FFN and
decode attention over a quantized KV cache.  Per-kernel lines take the median of five timed
graph replays.
cpu_baseline times the CPU oracle on the headline step (all host cores); cpu_baseline_1thread
the same on one thread; cpu_baseline_prefill the oracle on a sample of the prefill GEMM.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-weight GB/s (% HBM peak) at M=1 GEMV; TFLOP/s (% MFMA peak) at M=512"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_I8_PEAK_TOPS = 5000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def quantize_pack(q, torch, w: np.ndarray, bits: int, frac: float = 0.0, sym: bool = False, g: int = 128):
    n, k = w.shape
    dev = torch.device("cuda")
    d = q.desc(bits, n, k, group_size=g, zero_mode=q.QP_ZERO_MIDPOINT if sym else q.QP_ZERO_STORED)
    wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(dev)
    codes = torch.empty((n, k), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, k // g), dtype=torch.int16, device=dev)
    zeros = None if sym else torch.empty((n, k // g), dtype=torch.uint8, device=dev)
    kout = q.qp_outlier_count(n, k, frac)
    rowptr = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(kout, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(kout, 1), dtype=torch.int16, device=dev)
    wsb = q.qpack_quantize_workspace_bytes(d, frac)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _, nnz = q.qpack_quantize(d, wd, k, frac, codes, scales, zeros, rowptr, col, val, kout, ws, wsb)
    packed = torch.empty(q.qp_packed_bytes(d), dtype=torch.uint8, device=dev)
    q.qpack_pack(d, codes, packed)
    torch.cuda.synchronize()
    del wd, codes, ws
    return d, dict(packed=packed, scales=scales, zeros=zeros, rowptr=rowptr, col=col, val=val, nnz=nnz)


def quantize_pack_fp8(q, torch, w: np.ndarray, bits: int, g: int, sym: bool, fb_stride: int = 8):
    """fp8 scales with an fp16 fallback (qpack_quantize_fp8), packed in the device layout."""
    n, k = w.shape
    dev = torch.device("cuda")
    d = q.desc(bits, n, k, group_size=g, zero_mode=q.QP_ZERO_MIDPOINT if sym else q.QP_ZERO_STORED,
               scale_format=q.QP_SCALE_FP8)
    wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(dev)
    codes = torch.empty((n, k), dtype=torch.uint8, device=dev)
    wt = dict(sc8=torch.empty((n, k // g), dtype=torch.uint8, device=dev),
              zeros=None if sym else torch.empty((n, k // g), dtype=torch.uint8, device=dev),
              factors=torch.empty(n, dtype=torch.float32, device=dev),
              fb=torch.zeros((n, fb_stride), dtype=torch.int16, device=dev))
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    q.qpack_quantize_fp8(d, wd, k, codes, wt["sc8"], wt["zeros"], wt["factors"], wt["fb"], fb_stride, counts)
    wt["packed"] = torch.empty(q.qp_packed_bytes(d), dtype=torch.uint8, device=dev)
    q.qpack_pack(d, codes, wt["packed"])
    torch.cuda.synchronize()
    wt["fallbacks"] = int(counts.sum().item())
    del wd, codes
    return d, wt


def gemv_line_fp8(q, torch, stream, d, wt, nbytes, x, m, y, ldy):
    """gemv_line for a QP_SCALE_FP8 weight (its own clones for the >= 1 GiB rotation)."""
    fb_stride = wt["fb"].shape[1]
    keep = [{key: wt[key].clone() if wt[key] is not None else None for key in ("packed", "sc8", "zeros", "factors",
                                                                            "fb")}
            for _ in range(copies_for(nbytes))]
    hs = [q.weight_fp8(c["packed"], c["sc8"], c["factors"], c["fb"], fb_stride, c["zeros"]) for c in keep]
    k = d.k
    ms = time_graph(torch, lambda i: q.qlinear_gemv(d, hs[i % len(hs)], x, k, m, y, ldy), 2 * len(hs), stream)
    gbps = nbytes / (ms * 1e-3) / 1e9
    del hs, keep
    return dict(us=round(ms * 1e3, 3), GBps=round(gbps, 1), frac_hbm_peak=round(gbps / HBM_PEAK_GBS, 4),
                bytes=nbytes)


def weight_bytes(n: int, k: int, bits: int, nnz: int = 0, sym: bool = False, g: int = 128) -> int:
    """Algorithmic bytes a matmul must read for the weight: packed codes, fp16 scale and u8
    zero point per group of g (no zero point for symmetric groups), plus the outlier CSR
    (int32 col + fp16 val + rowptr)."""
    csr = (nnz * 6 + (n + 1) * 4) if nnz else 0
    return n * k * bits // 8 + (n * k // g) * (2 if sym else 3) + csr


def time_graph(torch, fn, reps: int, stream, trials: int = 5, warm_ms: float = 50.0) -> float:
    """Average ms of one fn(i) call: a graph of `reps` back-to-back calls (i = 0..reps-1), HIP
    events around each replay on the graph's stream; the median over `trials` replays, after
    about warm_ms of untimed replays (the clock settles under sustained load)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    for _ in range(min(500, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    del g
    return float(np.median(times))


ROTATION_BYTES = 1 << 30
CALLS = 100  # calls per timed graph replay for the compute-bound lines


def copies_for(nbytes: int, min_bytes: int = ROTATION_BYTES) -> int:
    """Distinct weight copies a memory-bound line rotates over: at least `min_bytes` in total
    (four times the 256 MB Infinity Cache), so each launch reads its weight from HBM."""
    return max(2, -(-min_bytes // nbytes))


GEMV_SOURCES = ("weight_only_mixed_amd/csrc/qmm_small.hip", "weight_only_mixed_amd/csrc/unpack.h",
                "weight_only_mixed_amd/csrc/qp_internal.h")
TRAFFIC_FILE = "profiles/pmc_traffic_gemv4096_gemm_prefill.md"


def gemv_kernel_name(bits: int, m: int, n: int) -> str:
    """Template instance qlinear_gemv launches for (bits, m, n) with groups of 128 and byte
    zero points: gemv_kernel<B, waves, ring depth, activation row pairs, group size, b-bit
    zero points> (the launcher in qmm_small.hip picks them the same way)."""
    mx = 1 if m <= 2 else 2 if m <= 4 else 4 if m <= 8 else 8
    nw = 4 if (n // 16 >= 512 or mx == 8) else 8
    return f"qp::gemv_kernel<{bits}, {nw}, 2, {mx}, 128, 0>"


def measured_traffic(kernel: str):
    """Per-launch HBM bytes of `kernel` from the committed FETCH_SIZE/WRITE_SIZE summary, or None
    if there is none or the GEMV sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    with open(path) as fh:
        for line in fh:
            mt = re.match(r"\s*traffic (.+) bytes=(\d+) csrc_sha256=([0-9a-f]+)\s*$", line)
            if mt and mt.group(1) == kernel and mt.group(3) == h.hexdigest():
                return int(mt.group(2))
    return None


def launch_floor_us(torch, stream, reps: int = 200) -> float:
    """Per-launch time of back-to-back dependent launches of a one-element fill kernel in one
    graph, timed like the GEMV: what every launch costs before it reads a byte."""
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    return time_graph(torch, lambda i: t.zero_(), reps, stream) * 1e3


def copy_gbps(torch, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy bandwidth (read + write bytes / time) of torch's copy kernel."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def pmc_pass(q, torch, workloads):
    """A short eager sequence for counter collection: the headline 4-bit M=1 GEMV and every
    (bits, M) GEMV of the sweep on four distinct weight copies each, the four batched stages of
    two Llama-7B stack layers (layer 5: 2-bit q/k/gate/up; layer 0: all 6-bit) on four copies
    each, the prefill GEMM twice (fp16 activations with
    outliers, then int8 activations), decode attention over two copies of
    the 32K MHA quantized cache, and a 1 GiB copy twice (the copy is the calibration kernel:
    its bytes are known)."""
    dev = torch.device("cuda")
    K = N = 4096
    d4, w4 = quantize_pack(q, torch, workloads.layer_weights(1), 4)
    h4 = [q.weight(w4["packed"].clone(), w4["scales"].clone(), w4["zeros"].clone()) for _ in range(4)]
    x1 = torch.from_numpy(workloads.activations_fp16(1, K, workloads.seed_for(1)).view(np.int16)).to(dev)
    y1 = torch.empty((1, N), dtype=torch.int16, device=dev)
    for h in h4:
        q.qlinear_gemv(d4, h, x1, K, 1, y1, N)
    torch.cuda.synchronize()
    del h4, w4
    w = workloads.layer_weights(2)
    for b in workloads.SWEEP_BITS:
        d, wt = quantize_pack(q, torch, w, b)
        hs = [q.weight(wt["packed"].clone(), wt["scales"].clone(), wt["zeros"].clone()) for _ in range(4)]
        for m in workloads.SWEEP_M:
            x = torch.from_numpy(workloads.activations_fp16(m, K, workloads.seed_for(2)).view(np.int16)).to(dev)
            y = torch.empty((m, N), dtype=torch.int16, device=dev)
            for h in hs:
                q.qlinear_gemv(d, h, x, K, m, y, N)
        torch.cuda.synchronize()
    xs = {k: torch.from_numpy(workloads.activations_fp16(1, k, workloads.seed_for(3)).view(np.int16)).to(dev)
          for k in (4096, 11008)}
    for layer in (5, 0):
        mats = {}
        for nm in workloads.LLAMA_MATRICES:
            n, k = workloads.STACK_SHAPES[nm]
            b = workloads.stack_bits(layer, nm)
            d, wt = quantize_pack(q, torch, workloads.weights_fp16(n, k, workloads.stack_matrix_seed(layer, nm)), b)
            mats[nm] = (d, [clone_weight(torch, wt) for _ in range(4)], n, k)
            del wt
        ys = {nm: torch.empty((1, mats[nm][2]), dtype=torch.int16, device=dev) for nm in mats}
        for stage in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            for c in range(4):
                q.qlinear_gemv_batch([q.gemv_problem(mats[nm][0], q.weight(mats[nm][1][c]["packed"],
                                                                           mats[nm][1][c]["scales"],
                                                                           mats[nm][1][c]["zeros"]),
                                                     xs[mats[nm][3]], mats[nm][3], 1, ys[nm], mats[nm][2])
                                      for nm in stage])
            torch.cuda.synchronize()
        del mats
    wp, _ = workloads.prefill_weights()
    dp, wt = quantize_pack(q, torch, wp, 4, workloads.PREFILL_OUTLIER_FRAC)
    hp = q.weight(wt["packed"], wt["scales"], wt["zeros"], wt["rowptr"], wt["col"], wt["val"], wt["nnz"])
    Mp, Kp, Np = workloads.PREFILL_M, workloads.PREFILL_K, workloads.PREFILL_N
    xp = torch.from_numpy(workloads.prefill_activations().view(np.int16)).to(dev)
    yp = torch.empty((Mp, Np), dtype=torch.int16, device=dev)
    wsb = q.qlinear_gemm_workspace_bytes(dp, Mp, wt["nnz"])
    wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
    for _ in range(2):
        q.qlinear_gemm(dp, hp, xp, Kp, Mp, yp, Np, wsp, wsb)
    torch.cuda.synchronize()
    del hp, wt, wsp
    dp, wt = quantize_pack(q, torch, wp, 4)  # integer-dot path on the same shape (no outliers)
    ha = q.weight(wt["packed"], wt["scales"], wt["zeros"])
    xq = torch.empty((Mp, Kp), dtype=torch.int8, device=dev)
    sx = torch.empty(Mp, dtype=torch.float32, device=dev)
    for _ in range(2):
        q.qact_quantize(xp, Kp, Mp, Kp, xq, sx)
        q.qlinear_gemm_a8(dp, ha, xq, sx, Mp, yp, Np)
    torch.cuda.synchronize()
    del ha, wt, xp, yp, xq, sx
    cfg = workloads.KV_MHA
    d = q.kv_desc(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["capacity"], 4, 8, 64, 64)
    rows = cfg["batch"] * cfg["kv_heads"] * cfg["capacity"]
    slots = torch.arange(rows, dtype=torch.int64, device=dev)
    cache = {}
    for w in (q.QKV_K, q.QKV_V):
        x = torch.from_numpy(workloads.kv_rows(rows, workloads.seed_for(6, 0, w)).view(np.int16)).to(dev)
        cache[w] = (torch.empty(q.qkv_cache_bytes(d, w), dtype=torch.uint8, device=dev),
                    torch.empty(q.qkv_scale_count(d, w), dtype=torch.float32, device=dev))
        q.qkv_quantize(d, w, x, 128, slots, rows, cache[w][0], cache[w][1])
        del x
    copies = [cache, {w: (c[0].clone(), c[1].clone()) for w, c in cache.items()}]
    qv = torch.from_numpy(workloads.kv_queries(cfg["batch"], cfg["q_heads"], workloads.seed_for(6) + 2)
                          .view(np.int16)).to(dev)
    ln = torch.full((cfg["batch"],), cfg["capacity"], dtype=torch.int32, device=dev)
    o = torch.empty((cfg["batch"], cfg["q_heads"], 128), dtype=torch.int16, device=dev)
    wsb = q.qattn_decode_workspace_bytes(d)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    for c in copies:
        q.qattn_decode(d, qv, c[q.QKV_K][0], c[q.QKV_K][1], c[q.QKV_V][0], c[q.QKV_V][1], ln, 1.0 / math.sqrt(128),
                       o, ws, wsb)
    torch.cuda.synchronize()
    del copies, cache
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("bench: pmc pass done")


def clone_weight(torch, wt):
    return dict(packed=wt["packed"].clone(), scales=wt["scales"].clone(),
                zeros=None if wt["zeros"] is None else wt["zeros"].clone())


def bench_stack(q, torch, workloads, stream, reps: int = 20):
    """Llama-7B-shaped 32-layer decode stack at M=1 (224 GEMVs per token, mixed bit table).
    One quantized template per (shape, bits) class, cloned so every matrix has its own HBM
    bytes (2.96 GB in total).  One token = per layer the four dependent stages [q, k, v], [o],
    [gate, up], [down], each one qlinear_gemv_batch launch (128 launches), in one HIP graph;
    also reported with one qlinear_gemv launch per matrix (224 launches)."""
    dev = torch.device("cuda")
    templates, mats, total = {}, [], 0
    for layer in range(workloads.STACK_LAYERS):
        for name in workloads.LLAMA_MATRICES:
            n, k = workloads.STACK_SHAPES[name]
            b = workloads.stack_bits(layer, name)
            key = (n, k, b)
            if key not in templates:
                w = workloads.weights_fp16(n, k, workloads.stack_matrix_seed(layer, name))
                templates[key] = quantize_pack(q, torch, w, b)
            d, wt = templates[key]
            c = clone_weight(torch, wt)
            mats.append((d, q.weight(c["packed"], c["scales"], c["zeros"]), c, n, k))
            total += weight_bytes(n, k, b)
    xs = {k: torch.from_numpy(workloads.activations_fp16(1, k, workloads.seed_for(3)).view(np.int16)).to(dev)
          for k in (4096, 11008)}
    ys = {n: torch.empty((1, n), dtype=torch.int16, device=dev) for n in (4096, 11008)}
    def token_us(g):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    # one launch per matrix
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=stream):
        for d, h, _, n, k in mats:
            q.qlinear_gemv(d, h, xs[k], k, 1, ys[n], n)
    us_each = token_us(g1)
    # one launch per dependent stage of a layer: [q, k, v], [o], [gate, up], [down]
    ys2 = {name: torch.empty((1, workloads.STACK_SHAPES[name][0]), dtype=torch.int16, device=dev)
           for name in workloads.LLAMA_MATRICES}
    stages = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=stream):
        for layer in range(workloads.STACK_LAYERS):
            byname = dict(zip(workloads.LLAMA_MATRICES, mats[7 * layer:7 * layer + 7]))
            for st in stages:
                probs = [q.gemv_problem(byname[nm][0], byname[nm][1], xs[byname[nm][4]], byname[nm][4], 1, ys2[nm],
                                        byname[nm][3]) for nm in st]
                q.qlinear_gemv_batch(probs)
    us = token_us(g2)
    gbps = total / (us * 1e-6) / 1e9
    bits_avg = sum(workloads.stack_bits(l, nm) * workloads.STACK_SHAPES[nm][0] * workloads.STACK_SHAPES[nm][1]
                   for l in range(workloads.STACK_LAYERS) for nm in workloads.LLAMA_MATRICES) / \
        sum(workloads.STACK_SHAPES[nm][0] * workloads.STACK_SHAPES[nm][1]
            for nm in workloads.LLAMA_MATRICES) / workloads.STACK_LAYERS
    del mats, templates
    return dict(us_per_token=round(us, 1), GBps=round(gbps, 1), frac_hbm_peak=round(gbps / HBM_PEAK_GBS, 4),
                bytes_per_token=total, launches_per_token=4 * workloads.STACK_LAYERS, avg_bits=round(bits_avg, 3),
                us_per_token_one_launch_per_matrix=round(us_each, 1),
                GBps_one_launch_per_matrix=round(total / (us_each * 1e-6) / 1e9, 1))


def bench_moe(q, torch, workloads, stream, reps: int = CALLS):
    """Routed-expert FFN: 16 experts x (gate, up 14336x4096; down 4096x14336), 4-bit, 128 tokens
    top-2 with Zipf(1.1) routing, one qmoe_ffn call.  One quantized template per matrix kind,
    cloned per expert (1.48 GB of expert weights); gate and up rows interleaved per 16-row block
    for the SwiGLU epilogue."""
    dev = torch.device("cuda")
    E, D, F, T, K = (workloads.MOE_EXPERTS, workloads.MOE_DMODEL, workloads.MOE_DFF, workloads.MOE_TOKENS,
                     workloads.MOE_TOPK)
    g, u, dn = workloads.moe_expert(0)
    gu = workloads.interleave_row_blocks(g, u, 16)
    d_gu, t_gu = quantize_pack(q, torch, gu, 4)
    d_dn, t_dn = quantize_pack(q, torch, dn, 4)
    del g, u, dn, gu
    keep, h_gu, h_dn = [], [], []
    for _ in range(E):
        a, b = clone_weight(torch, t_gu), clone_weight(torch, t_dn)
        keep += [a, b]
        h_gu.append(q.weight(a["packed"], a["scales"], a["zeros"]))
        h_dn.append(q.weight(b["packed"], b["scales"], b["zeros"]))
    x, ids, wts = workloads.moe_inputs()
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    idd = torch.from_numpy(ids.astype(np.int32)).to(dev)
    wtd = torch.from_numpy(wts.astype(np.float32)).to(dev)
    out = torch.empty((T, D), dtype=torch.int16, device=dev)
    wsb = q.qmoe_ffn_workspace_bytes(T, K, E, D, F)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    fn = lambda i: q.qmoe_ffn(d_gu, h_gu, d_dn, h_dn, xd, D, T, idd, wtd, K, out, D, ws, wsb)
    ms = time_graph(torch, fn, reps, stream)
    active = int((np.bincount(ids.ravel(), minlength=E) > 0).sum())
    wbytes = active * (weight_bytes(2 * F, D, 4) + weight_bytes(D, F, 4))
    flops = 2 * T * K * (2 * F * D + D * F)
    return dict(us=round(ms * 1e3, 1), GBps=round(wbytes / (ms * 1e-3) / 1e9, 1),
                frac_hbm_peak=round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                TFLOPs=round(flops / (ms * 1e-3) / 1e12, 2), active_experts=active, weight_bytes=wbytes)


def kv_call_bytes(q, d, lens) -> int:
    """Algorithmic bytes of one decode-attention call: the K and V codes and fp32 scales of the
    first lens[b] tokens of every (sequence, kv head); queries and outputs (a few KB) left out."""
    per_tok = (128 * d.k_bits // 8 + 4 * (128 // d.k_group) + 128 * d.v_bits // 8 + 4 * (128 // d.v_group))
    return int(sum(int(L) for L in lens)) * d.kv_heads * per_tok


def bench_kv(q, torch, workloads, stream, min_bytes: int = 1 << 30):
    """Decode attention over the quantized KV cache (groups of 64, fp32 scales): INT4 K with
    INT8 V on the KV page's 7B MHA layer at a 32K context and on a GQA layer with four 8K
    sequences, and the MHA layer all INT8 and all INT4.  Each layer's cache is quantized once through qkv_quantize; the timed graph
    rotates over enough distinct layer caches (>= 1 GiB) that the cache streams from HBM."""
    out = {}
    for key, name, kb, vb in (("kv_mha", "KV_MHA", 4, 8), ("kv_gqa", "KV_GQA", 4, 8), ("kv_mha_k8v8", "KV_MHA", 8, 8),
                              ("kv_mha_k4v4", "KV_MHA", 4, 4)):
        cfg = getattr(workloads, name)
        d = q.kv_desc(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["capacity"], kb, vb, 64, 64)
        rows = cfg["batch"] * cfg["kv_heads"] * cfg["capacity"]
        lens = np.full(cfg["batch"], cfg["capacity"], np.int32)
        nbytes = kv_call_bytes(q, d, lens)
        layers = max(2, -(-min_bytes // nbytes))
        slots = torch.arange(rows, dtype=torch.int64, device="cuda")
        caches = []
        for layer in range(layers):
            c = {}
            for w in (q.QKV_K, q.QKV_V):
                if layer == 0:
                    x = torch.from_numpy(workloads.kv_rows(rows, workloads.seed_for(6, 0, w)).view(np.int16)).cuda()
                    c[w] = (torch.empty(q.qkv_cache_bytes(d, w), dtype=torch.uint8, device="cuda"),
                            torch.empty(q.qkv_scale_count(d, w), dtype=torch.float32, device="cuda"))
                    q.qkv_quantize(d, w, x, 128, slots, rows, c[w][0], c[w][1])
                    del x
                else:
                    c[w] = (caches[0][w][0].clone(), caches[0][w][1].clone())
            caches.append(c)
        qv = torch.from_numpy(workloads.kv_queries(cfg["batch"], cfg["q_heads"], workloads.seed_for(6) + 2)
                              .view(np.int16)).cuda()
        ln = torch.from_numpy(lens).cuda()
        o = torch.empty((cfg["batch"], cfg["q_heads"], 128), dtype=torch.int16, device="cuda")
        wsb = q.qattn_decode_workspace_bytes(d)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        sm = 1.0 / math.sqrt(128)

        def call(i):
            c = caches[i % layers]
            q.qattn_decode(d, qv, c[q.QKV_K][0], c[q.QKV_K][1], c[q.QKV_V][0], c[q.QKV_V][1], ln, sm, o, ws, wsb)

        ms = time_graph(torch, call, 2 * layers, stream)
        flops = 4 * int(lens.sum()) * cfg["q_heads"] * 128
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[key] = dict(us=round(ms * 1e3, 2), GBps=round(gbps, 1), frac_hbm_peak=round(gbps / HBM_PEAK_GBS, 4),
                        TFLOPs=round(flops / (ms * 1e-3) / 1e12, 2), bytes=nbytes, layers_rotated=layers,
                        shape=dict(batch=cfg["batch"], q_heads=cfg["q_heads"], kv_heads=cfg["kv_heads"],
                                   tokens=cfg["capacity"], k_bits=kb, v_bits=vb, group=64),
                        kernel=f"qp::kv_attn_kernel<{kb}, {vb}, 64, 64>")
        del caches, o, ws
    return out


def rotated_gemv(q, torch, d, wt, nbytes):
    """Handles of enough clones of one packed weight for a >= 1 GiB rotation (the clones are
    kept alive by the returned list)."""
    n = copies_for(nbytes)
    keep = [clone_weight(torch, wt) for _ in range(n)]
    return [q.weight(c["packed"], c["scales"], c["zeros"]) for c in keep], keep


def gemv_line(q, torch, stream, d, wt, nbytes, x, m, y, ldy):
    """Median-of-5 time of one qlinear_gemv launch over a >= 1 GiB rotation."""
    hs, keep = rotated_gemv(q, torch, d, wt, nbytes)
    k = d.k
    ms = time_graph(torch, lambda i: q.qlinear_gemv(d, hs[i % len(hs)], x, k, m, y, ldy), 2 * len(hs), stream)
    gbps = nbytes / (ms * 1e-3) / 1e9
    del hs, keep
    return dict(us=round(ms * 1e3, 3), GBps=round(gbps, 1), frac_hbm_peak=round(gbps / HBM_PEAK_GBS, 4),
                bytes=nbytes)


def bench_prefill(q, torch, workloads, stream):
    """Prefill dequant-GEMM (M=512, K=8192, N=28672, 4-bit g=128, 0.1% fp16 CSR outliers), end to
    end through qlinear_gemm, and the same weight without its outliers (the dense kernel
    alone).  The weight (123 MB) is read once per launch; its reuse across the 512 rows makes
    the call MFMA-bound, so no rotation is needed."""
    dev = torch.device("cuda")
    wp, _ = workloads.prefill_weights()
    dp, wt = quantize_pack(q, torch, wp, 4, workloads.PREFILL_OUTLIER_FRAC)
    del wp
    Mp, Kp, Np = workloads.PREFILL_M, workloads.PREFILL_K, workloads.PREFILL_N
    hp = q.weight(wt["packed"], wt["scales"], wt["zeros"], wt["rowptr"], wt["col"], wt["val"], wt["nnz"])
    hd = q.weight(wt["packed"], wt["scales"], wt["zeros"])
    xp = torch.from_numpy(workloads.prefill_activations().view(np.int16)).to(dev)
    yp = torch.empty((Mp, Np), dtype=torch.int16, device=dev)
    wsb = q.qlinear_gemm_workspace_bytes(dp, Mp, wt["nnz"])
    wsp = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    ms = time_graph(torch, lambda i: q.qlinear_gemm(dp, hp, xp, Kp, Mp, yp, Np, wsp, wsb), CALLS, stream)
    ms_dense = time_graph(torch, lambda i: q.qlinear_gemm(dp, hd, xp, Kp, Mp, yp, Np, None, 0), CALLS, stream)
    # one GPU's share under 8-way column parallelism: the first N/8 rows of the same quantized
    # weight with their outliers; with the split workspace (k in parts) and without
    ns = Np // 8
    ds = q.desc(4, ns, Kp, q.QP_LAYOUT_DEVICE)
    nnz_s = int(wt["rowptr"][ns].item())
    hs = q.weight(wt["packed"], wt["scales"], wt["zeros"], wt["rowptr"], wt["col"], wt["val"], nnz_s)
    ys = torch.empty((Mp, ns), dtype=torch.int16, device=dev)
    wsb_s = q.qlinear_gemm_workspace_bytes(ds, Mp, nnz_s)
    wsb_o = (2 * Kp + 4 * ns) * ((Mp + 127) // 128 * 128)  # the outlier part alone: no split
    ws_s = torch.empty(wsb_s, dtype=torch.uint8, device=dev)
    ms_s = time_graph(torch, lambda i: q.qlinear_gemm(ds, hs, xp, Kp, Mp, ys, ns, ws_s, wsb_s), CALLS, stream)
    ms_u = time_graph(torch, lambda i: q.qlinear_gemm(ds, hs, xp, Kp, Mp, ys, ns, ws_s, wsb_o), CALLS, stream)
    fl_s = 2 * Mp * ns * Kp + 2 * Mp * nnz_s
    shard = dict(shape=dict(m=Mp, k=Kp, n=ns, nnz=nnz_s), k_parts=(wsb_s - wsb_o) // (4 * Mp * ns) if wsb_s > wsb_o else 1,
                 us=round(ms_s * 1e3, 2), TFLOPs=round(fl_s / (ms_s * 1e-3) / 1e12, 1),
                 frac_mfma_peak=round(fl_s / (ms_s * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                 unsplit_us=round(ms_u * 1e3, 2),
                 unsplit_TFLOPs=round(fl_s / (ms_u * 1e-3) / 1e12, 1))
    del ws_s, ys
    dense_flops = 2 * Mp * Np * Kp
    flops = dense_flops + 2 * Mp * wt["nnz"]
    tf = flops / (ms * 1e-3) / 1e12
    tf_dense = dense_flops / (ms_dense * 1e-3) / 1e12
    wbytes = weight_bytes(Np, Kp, 4, wt["nnz"])
    del hp, hd, wt, xp, yp, wsp
    roof = dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(tf / MFMA_F16_PEAK_TFLOPS, 4), traffic=None,
                kernel="qlinear_gemm end to end (config M=512 K=8192 N=28672, 4-bit + outliers)",
                flops_per_launch=flops, avg_launch_us=round(ms * 1e3, 2),
                dense_kernel_alone=dict(achieved=round(tf_dense, 1), frac=round(tf_dense / MFMA_F16_PEAK_TFLOPS, 4),
                                        avg_launch_us=round(ms_dense * 1e3, 2), flops_per_launch=dense_flops,
                                        kernel="qp::gemm_kernel<4, 0, 8> (no outliers)"),
                weight_bytes=wbytes, tp8_shard=shard)
    return roof


def bench_gemv_large(q, torch, workloads, stream):
    """Decode GEMV on the prefill case's 70B-style FFN weight (N=28672, K=8192, 4-bit g=128, no
    outliers: 124 MB with its metadata) at M = 1 and 8, over a >= 1 GiB rotation: the kernel's
    streaming rate once one launch carries enough bytes to hide the launch and its first
    fetches."""
    dev = torch.device("cuda")
    wp, _ = workloads.prefill_weights()
    dp, wt = quantize_pack(q, torch, wp, 4)
    del wp
    N, K = workloads.PREFILL_N, workloads.PREFILL_K
    nb = weight_bytes(N, K, 4)
    out = {}
    for m in (1, 8):
        x = torch.from_numpy(workloads.activations_fp16(m, K, workloads.seed_for(4)).view(np.int16)).to(dev)
        y = torch.empty((m, N), dtype=torch.int16, device=dev)
        line = gemv_line(q, torch, stream, dp, wt, nb, x, m, y, N)
        line["kernel"] = gemv_kernel_name(4, m, N)
        out[f"n{N}_k{K}_b4_m{m}"] = line
    del wt
    return out


def bench_prefill_variants(q, torch, workloads, stream):
    """The prefill GEMM (M=512, K=8192, N=28672, no outliers) for the metadata variants of the
    mixed-bit page (s2.3): groups of 64 and 32, symmetric groups, zero points in b bits, fp8
    scales with an fp16 fallback."""
    dev = torch.device("cuda")
    wp, _ = workloads.prefill_weights()
    Mp, Kp, Np = workloads.PREFILL_M, workloads.PREFILL_K, workloads.PREFILL_N
    xp = torch.from_numpy(workloads.prefill_activations().view(np.int16)).to(dev)
    yp = torch.empty((Mp, Np), dtype=torch.int16, device=dev)
    out = {}
    for bits, g, sym, packed in ((4, 128, False, True), (4, 64, False, False), (2, 32, False, False),
                                 (2, 32, False, True), (2, 32, True, False), (5, 64, False, True)):
        d, wt = quantize_pack(q, torch, wp, bits, sym=sym, g=g)
        z = wt["zeros"]
        if packed:
            d = q.desc(bits, Np, Kp, group_size=g, zero_mode=q.QP_ZERO_PACKED)
            z = torch.empty(q.qp_zero_bytes(d), dtype=torch.uint8, device=dev)
            q.qpack_pack_zeros(d, wt["zeros"], z)
        h = q.weight(wt["packed"], wt["scales"], z)
        ms = time_graph(torch, lambda i: q.qlinear_gemm(d, h, xp, Kp, Mp, yp, Np, None, 0), CALLS, stream)
        tf = 2 * Mp * Np * Kp / (ms * 1e-3) / 1e12
        key = f"b{bits}_g{g}" + ("_sym" if sym else "") + ("_bbit_zeros" if packed else "")
        out[key] = dict(us=round(ms * 1e3, 2), TFLOPs=round(tf, 1), frac_mfma_peak=round(tf / MFMA_F16_PEAK_TFLOPS, 4))
        del wt, h, z
    for bits, g, sym in ((2, 32, True), (4, 128, False)):  # fp8 scales with an fp16 fallback
        d, wt = quantize_pack_fp8(q, torch, wp, bits, g, sym)
        h = q.weight_fp8(wt["packed"], wt["sc8"], wt["factors"], wt["fb"], wt["fb"].shape[1], wt["zeros"])
        ms = time_graph(torch, lambda i: q.qlinear_gemm(d, h, xp, Kp, Mp, yp, Np, None, 0), CALLS, stream)
        tf = 2 * Mp * Np * Kp / (ms * 1e-3) / 1e12
        out[f"b{bits}_g{g}" + ("_sym" if sym else "") + "_fp8_scales"] = dict(
            us=round(ms * 1e3, 2), TFLOPs=round(tf, 1), frac_mfma_peak=round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            fallback_groups=wt["fallbacks"])
        del wt, h
    del xp, yp
    return out


def bench_prefill_a8(q, torch, workloads, stream):
    """Integer-dot prefill (the W8A8 path): the prefill shape M=512, K=8192, N=28672 at 4 bits,
    g=128, on int8 activations (no outlier add-back: the held-out weights stay in their groups
    here).  Timed as the GEMM alone (qlinear_gemm_a8 on int8 activations already resident) and
    end to end (qact_quantize of the fp16 activations, then the GEMM); ops = 2 M N K against
    the dense int8 matrix-core peak."""
    dev = torch.device("cuda")
    wp, _ = workloads.prefill_weights()
    dp, wt = quantize_pack(q, torch, wp, 4)
    del wp
    Mp, Kp, Np = workloads.PREFILL_M, workloads.PREFILL_K, workloads.PREFILL_N
    h = q.weight(wt["packed"], wt["scales"], wt["zeros"])
    xp = torch.from_numpy(workloads.prefill_activations().view(np.int16)).to(dev)
    xq = torch.empty((Mp, Kp), dtype=torch.int8, device=dev)
    sx = torch.empty(Mp, dtype=torch.float32, device=dev)
    yp = torch.empty((Mp, Np), dtype=torch.int16, device=dev)
    q.qact_quantize(xp, Kp, Mp, Kp, xq, sx)
    ms_gemm = time_graph(torch, lambda i: q.qlinear_gemm_a8(dp, h, xq, sx, Mp, yp, Np), CALLS, stream)

    def e2e(i):
        q.qact_quantize(xp, Kp, Mp, Kp, xq, sx)
        q.qlinear_gemm_a8(dp, h, xq, sx, Mp, yp, Np)

    ms_e2e = time_graph(torch, e2e, CALLS, stream)
    ms_act = time_graph(torch, lambda i: q.qact_quantize(xp, Kp, Mp, Kp, xq, sx), CALLS, stream)
    ops = 2 * Mp * Np * Kp
    tops = ops / (ms_gemm * 1e-3) / 1e12
    tops_e2e = ops / (ms_e2e * 1e-3) / 1e12
    del h, wt, xp, xq, sx, yp
    return dict(bound="mfma", achieved=round(tops, 1), peak=MFMA_I8_PEAK_TOPS, unit="TOP/s",
                frac=round(tops / MFMA_I8_PEAK_TOPS, 4), traffic=None,
                kernel="qp::gemm_a8_kernel<4> (M=512 K=8192 N=28672, 4-bit g=128, int8 activations)",
                ops_per_launch=ops, avg_launch_us=round(ms_gemm * 1e3, 2),
                end_to_end=dict(achieved=round(tops_e2e, 1), frac=round(tops_e2e / MFMA_I8_PEAK_TOPS, 4),
                                avg_us=round(ms_e2e * 1e3, 2), kernels="qact_quantize + qlinear_gemm_a8"),
                act_quantize_us=round(ms_act * 1e3, 2),
                act_quantize_GBps=round((Mp * Kp * 3 + Mp * 4) / (ms_act * 1e-3) / 1e9, 1))


def host_read_gbps(nbytes: int = 1 << 30, threads: int = 0) -> float:
    """Host memory read bandwidth: numpy sums over slices of a 1 GiB array in parallel threads
    (the reductions release the GIL), the reference for the host GEMV's GB/s."""
    from concurrent.futures import ThreadPoolExecutor
    n = threads or max(1, (os.cpu_count() or 2) - 1)
    a = np.ones(nbytes // 8, np.uint64)
    parts = np.array_split(a, n)
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(lambda p: int(p.sum()), parts))
        t = time.perf_counter()
        for _ in range(3):
            list(ex.map(lambda p: int(p.sum()), parts))
        dt = (time.perf_counter() - t) / 3
    return nbytes / dt / 1e9


def bench_host_gemv(q, workloads, K, N):
    """Host fused unpack-MAC GEMV (canonical layout, the CPU half of a layer split) on the 4096 x
    4096 layer at M = 1, rotating over >= 1 GiB of weight copies; GB/s of packed bytes."""
    import oracle  # the oracle only quantizes and packs the inputs here
    out = {}
    w = workloads.layer_weights(1)
    x = np.ascontiguousarray(workloads.activations_fp16(1, K, workloads.seed_for(1))).view(np.uint16)
    y = np.zeros((1, N), np.uint16)
    for bits in (2, 4, 6):
        r = oracle.quantize(w, bits)
        packed = np.ascontiguousarray(oracle.pack_canonical(r["codes"], bits))
        sc, z = np.ascontiguousarray(r["scales"]), np.ascontiguousarray(r["zeros"])
        nb = weight_bytes(N, K, bits)
        copies = [(packed.copy(), sc.copy(), z.copy()) for _ in range(copies_for(nb))]
        hs = [q.qp_weight(p.ctypes.data, s_.ctypes.data, z_.ctypes.data, None, None, None, 0) for p, s_, z_ in copies]
        d = q.desc(bits, N, K, q.QP_LAYOUT_CANONICAL)
        for h in hs[:4]:
            q.qlinear_gemv_host(d, h, x, K, 1, y, N)
        times = []
        for _ in range(3):
            t = time.perf_counter()
            for h in hs:
                q.qlinear_gemv_host(d, h, x, K, 1, y, N)
            times.append((time.perf_counter() - t) / len(hs))
        dt = float(np.median(times))
        out[f"b{bits}_m1"] = dict(us=round(dt * 1e6, 1), GBps=round(nb / dt / 1e9, 2), bytes=nb, copies=len(hs))
        del copies, hs
    out["isa"] = q.qlinear_gemv_host_isa()
    if out["isa"] == "avx512vbmi":  # the AVX2 path beside it, on the 4-bit layer
        os.environ["QPACK_HOST_AVX2"] = "1"
        try:
            r = oracle.quantize(w, 4)
            p_, s_, z_ = (np.ascontiguousarray(a) for a in (oracle.pack_canonical(r["codes"], 4), r["scales"], r["zeros"]))
            h = q.qp_weight(p_.ctypes.data, s_.ctypes.data, z_.ctypes.data, None, None, None, 0)
            d = q.desc(4, N, K, q.QP_LAYOUT_CANONICAL)
            copies = [(p_.copy(), s_.copy(), z_.copy()) for _ in range(copies_for(p_.nbytes))]
            hs = [q.qp_weight(a.ctypes.data, b.ctypes.data, c.ctypes.data, None, None, None, 0) for a, b, c in copies]
            for h in hs[:4]:
                q.qlinear_gemv_host(d, h, x, K, 1, y, N)
            t = time.perf_counter()
            for h in hs:
                q.qlinear_gemv_host(d, h, x, K, 1, y, N)
            dt = (time.perf_counter() - t) / len(hs)
            out["b4_m1_avx2"] = dict(us=round(dt * 1e6, 1), GBps=round(p_.nbytes / dt / 1e9, 2))
            del copies, hs
        finally:
            del os.environ["QPACK_HOST_AVX2"]
    out["threads"] = max(1, (os.cpu_count() or 2) - 1)
    out["host_read_GBps"] = round(host_read_gbps(), 2)
    return out


def cpu_baselines(workloads, K, N, headline_bytes, seconds):
    """The oracle (as it stands) on the host cores: the headline GEMV repeated for about
    `seconds`, the same on one thread, and a column sample of the prefill GEMM in fp64."""
    import oracle
    w = workloads.layer_weights(1)
    ref = oracle.quantize(w, 4)
    x = workloads.activations_fp16(1, K, workloads.seed_for(1))
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.linear(x, ref)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    cpu = dict(value=round(headline_bytes * reps / dt / 1e9, 4), unit="GB/s", cores=cores, kind="oracle",
               sample=f"{reps} headline steps (fp64 GEMV, 4096x4096 4-bit, M=1, over the oracle's own codes), "
                      f"{dt:.1f} s")
    oracle.set_num_threads(1)
    t0 = time.perf_counter()
    reps1 = 0
    while time.perf_counter() - t0 < seconds / 4:
        oracle.linear(x, ref)
        reps1 += 1
    dt1 = time.perf_counter() - t0
    oracle.set_num_threads(cores)
    cpu1 = dict(value=round(headline_bytes * reps1 / dt1 / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{reps1} headline steps on one thread, {dt1:.1f} s")
    # prefill: every activation row against a sample of weight rows (columns of y)
    wp, _ = workloads.prefill_weights()
    ncols = 512
    refp = oracle.quantize(np.ascontiguousarray(wp[:ncols]), 4)
    del wp
    xp = workloads.prefill_activations()
    t0 = time.perf_counter()
    oracle.linear(xp, refp)
    dtp = time.perf_counter() - t0
    flops = 2 * xp.shape[0] * ncols * xp.shape[1]
    cpup = dict(value=round(flops / dtp / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"all {xp.shape[0]} activation rows x {ncols} of the 28672 weight rows of the prefill "
                       f"GEMM (K={xp.shape[1]}, fp64, outliers not held out in the sample), {dtp:.1f} s")
    return cpu, cpu1, cpup


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baselines")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=512 GEMM line")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 2/3/5/6-bit x M=1,4,8 sweep lines")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the symmetric / small-group / b-bit zero point GEMV lines")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer decode stack line")
    ap.add_argument("--no-moe", action="store_true", help="skip the routed-expert FFN line")
    ap.add_argument("--no-kv", action="store_true", help="skip the quantized-KV decode attention line")
    ap.add_argument("--no-host", action="store_true", help="skip the host (CPU) fused GEMV line")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="eager launches only (the headline GEMV, each GEMV of the sweep, the prefill GEMM, "
                         "decode attention, a 1 GiB copy) for hardware-counter runs; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", flush=True)
        sys.exit(2)

    import torch

    import weight_only_mixed_amd as q
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    K = N = 4096

    if args.pmc_pass:
        pmc_pass(q, torch, workloads)
        return

    # ---- headline: 4096 x 4096, 4-bit, M = 1 ------------------------------------------------
    log("bench: quantize + pack the 4096x4096 4-bit layer")
    d4, w4 = quantize_pack(q, torch, workloads.layer_weights(1), 4)
    step_bytes = weight_bytes(N, K, 4)
    h4, keep4 = rotated_gemv(q, torch, d4, w4, step_bytes)
    ncopies = len(h4)
    x1 = torch.from_numpy(workloads.activations_fp16(1, K, workloads.seed_for(1)).view(np.int16)).to(dev)
    y1 = torch.empty((1, N), dtype=torch.int16, device=dev)
    log(f"bench: {ncopies} copies, {ncopies * step_bytes / 2**30:.2f} GiB of packed weights")
    stream = torch.cuda.Stream()

    def capture(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                q.qlinear_gemv(d4, h4[i % ncopies], x1, K, 1, y1, N)
        return g

    g_full = capture(ncopies)
    rem = args.steps % ncopies
    g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(-(-args.warmup // ncopies)):
        g_full.replay()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps // ncopies):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    value = step_bytes * args.steps / (ms_total * 1e-3) / 1e9
    kname = gemv_kernel_name(4, 1, N)
    roofline = dict(bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(value / HBM_PEAK_GBS, 4), traffic=measured_traffic(kname),
                    kernel=kname, bytes_per_launch=step_bytes, avg_launch_us=round(ms_per_step * 1e3, 3))
    del g_full, g_rem
    floor_us = launch_floor_us(torch, stream)
    # the launch floor bounds a 4096x4096 launch: bytes / (floor + bytes at peak)
    roofline["launch_floor_us"] = round(floor_us, 3)
    roofline["frac_of_launch_bound"] = round(
        value / (step_bytes / ((floor_us + step_bytes / HBM_PEAK_GBS / 1e3) * 1e-6) / 1e9), 4)
    extra = {"gemv_4096_4bit_m1_median5": gemv_line(q, torch, stream, d4, w4, step_bytes, x1, 1, y1, N)}
    del h4, keep4

    if not args.no_prefill:
        log("bench: prefill GEMM M=512 K=8192 N=28672 4-bit + 0.1% outliers")
        extra["roofline_prefill"] = bench_prefill(q, torch, workloads, stream)
        log("bench: decode GEMV on the same 28672x8192 4-bit weight, M=1 and 8")
        extra["gemv_large_70b_ffn"] = bench_gemv_large(q, torch, workloads, stream)
        log("bench: integer-dot prefill (int8 activations) M=512 K=8192 N=28672 4-bit")
        extra["roofline_prefill_a8"] = bench_prefill_a8(q, torch, workloads, stream)
        if not args.no_variants:
            log("bench: prefill GEMM metadata variants (groups of 64/32, symmetric, b-bit zero points)")
            extra["prefill_variants"] = bench_prefill_variants(q, torch, workloads, stream)

    if not args.no_sweep:
        log("bench: 4096x4096 sweep, bits 2/3/5/6 x M 1/4/8")
        sweep = {}
        w2 = workloads.layer_weights(2)
        for b in workloads.SWEEP_BITS:
            d, wt = quantize_pack(q, torch, w2, b)
            for m in workloads.SWEEP_M:
                x = torch.from_numpy(workloads.activations_fp16(m, K, workloads.seed_for(2)).view(np.int16)).to(dev)
                y = torch.empty((m, N), dtype=torch.int16, device=dev)
                line = gemv_line(q, torch, stream, d, wt, weight_bytes(N, K, b), x, m, y, N)
                line["kernel"] = gemv_kernel_name(b, m, N)
                sweep[f"b{b}_m{m}"] = line
            del wt
        extra["sweep_4096"] = sweep

    if not args.no_variants:
        log("bench: 4096x4096 GEMV at M=1: symmetric groups, groups of 32/64, b-bit zero points")
        w2 = workloads.layer_weights(2)
        sym = {}
        for b in (2, 3):
            ds, wsy = quantize_pack(q, torch, w2, b, sym=True)
            sym[f"b{b}_m1"] = gemv_line(q, torch, stream, ds, wsy, weight_bytes(N, K, b, sym=True), x1, 1, y1, N)
            del wsy
        extra["gemv_4096_sym_m1"] = sym
        small = {}
        for b, g, sy in ((2, 32, True), (2, 64, True), (2, 32, False), (5, 64, False), (6, 64, False)):
            ds, wsy = quantize_pack(q, torch, w2, b, sym=sy, g=g)
            bs = weight_bytes(N, K, b, sym=sy, g=g)
            line = gemv_line(q, torch, stream, ds, wsy, bs, x1, 1, y1, N)
            line["bits_per_weight"] = round(8 * bs / (N * K), 4)
            small[f"b{b}_g{g}{'_sym' if sy else ''}"] = line
            del wsy
        extra["gemv_4096_small_groups_m1"] = small
        pz = {}
        for b, g in ((2, 32), (3, 64), (5, 64), (6, 128)):
            dz = q.desc(b, N, K, group_size=g, zero_mode=q.QP_ZERO_PACKED)
            _, wz = quantize_pack(q, torch, w2, b, g=g)
            zp = torch.empty(q.qp_zero_bytes(dz), dtype=torch.uint8, device=dev)
            q.qpack_pack_zeros(dz, wz["zeros"], zp)
            wz["zeros"] = zp
            bz = N * K * b // 8 + (N * K // g) * 2 + q.qp_zero_bytes(dz)
            line = gemv_line(q, torch, stream, dz, wz, bz, x1, 1, y1, N)
            line["bits_per_weight"] = round(8 * bz / (N * K), 4)
            pz[f"b{b}_g{g}"] = line
            del wz, zp
        extra["gemv_4096_packed_zeros_m1"] = pz
        log("bench: 4096x4096 GEMV with fp8 scales (fp16 fallback), M=1 and 16")
        f8 = {}
        x16 = torch.from_numpy(workloads.activations_fp16(16, K, workloads.seed_for(2)).view(np.int16)).to(dev)
        y16 = torch.empty((16, N), dtype=torch.int16, device=dev)
        for b, g, sy in ((2, 32, True), (3, 64, True), (4, 128, False)):
            d8, w8 = quantize_pack_fp8(q, torch, w2, b, g, sy)
            # codes, one scale byte per group, zero-point bytes unless symmetric, one fp32 factor per row
            b8 = N * K * b // 8 + (N * K // g) * (1 if sy else 2) + 4 * N
            for m, x, y in ((1, x1, y1), (16, x16, y16)):
                line = gemv_line_fp8(q, torch, stream, d8, w8, b8, x, m, y, N)
                line["bits_per_weight"] = round(8 * b8 / (N * K), 4)
                line["fallback_groups"] = w8["fallbacks"]
                f8[f"b{b}_g{g}{'_sym' if sy else ''}_m{m}"] = line
            del w8
        extra["gemv_4096_fp8_scales"] = f8
    if not args.no_stack:
        log("bench: Llama-7B-shaped 32-layer decode stack at M=1")
        extra["stack_llama7b_m1"] = bench_stack(q, torch, workloads, stream)
    if not args.no_moe:
        log("bench: routed-expert FFN, 16 experts, 128 tokens top-2")
        extra["moe_16x_ffn_t128"] = bench_moe(q, torch, workloads, stream)
    if not args.no_kv:
        log("bench: decode attention over an INT4-K / INT8-V cache (32K MHA, 4 x 8K GQA)")
        extra["kv_decode_attention"] = bench_kv(q, torch, workloads, stream)

    if not args.no_host:
        log("bench: host fused unpack-MAC GEMV, 4096x4096, M=1")
        extra["host_gemv_4096_m1"] = bench_host_gemv(q, workloads, K, N)

    log("bench: 1 GiB device copy")
    extra["copy_GBps"] = round(copy_gbps(torch), 1)

    cpu = cpu1 = cpup = None
    if not args.no_cpu:
        log("bench: CPU oracle baselines")
        cpu, cpu1, cpup = cpu_baselines(workloads, K, N, step_bytes, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "4096x4096 layer, 4-bit asymmetric g=128, decode M=1 GEMV (page units, "
                               "device tile layout)",
                   "bits": 4, "m": 1, "n": N, "k": K, "group": 128,
                   "weight_copies": ncopies, "step_weight_bytes": step_bytes,
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "cpu_baseline_prefill": cpup,
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
