"""Benchmark: weight-only mixed-bit decode GEMV on one MI355X.

Workload (one "step"): the 4096 x 4096 layer at 2, 3, 5 and 6 bits (asymmetric, groups of
128 along K, page packing units) times decode batches M = 1, 4, 8 -- twelve qlinear_gemv
calls.  Weights are quantized and packed once (the offline repack of the 70B page, s3) and
the step rotates over enough identical copies (>= 1 GB in total) that every weight byte is
read from HBM, as in a real decode pass over distinct layers, not from the 256 MB
Infinity Cache.  Each step is one captured HIP graph, replayed.

value = packed-weight bytes (codes + fp16 scales + u8 zero points) of the step / step time.
The roofline object covers the kernel with the largest share of the step, timed live with
HIP events around a graph of back-to-back launches on its own stream.  A secondary line
measures the prefill dequant-GEMM (M=512, K=8192, N=28672, 4-bit + 0.1% outliers) in
TFLOP/s.  Further lines: the 4-bit 4096 x 4096 GEMV at M=1, the same layer at 2 and 3 bits
with symmetric groups (no zero points), with groups of 32 and 64, and with zero points kept in
b bits, a Llama-7B-shaped decode stack, a 16-expert FFN, and decode attention over a quantized
KV cache.
cpu_baseline times the CPU oracle on the same step; cpu_baseline_1thread times one step of it on
one thread.
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


def weight_bytes(n: int, k: int, bits: int, nnz: int = 0, sym: bool = False, g: int = 128) -> int:
    """Algorithmic bytes a matmul must read for the weight: packed codes, fp16 scale and u8
    zero point per group of g (no zero point for symmetric groups), plus the outlier CSR
    (int32 col + fp16 val + rowptr)."""
    csr = (nnz * 6 + (n + 1) * 4) if nnz else 0
    return n * k * bits // 8 + (n * k // g) * (2 if sym else 3) + csr


def time_graph(torch, fn, reps: int, stream) -> float:
    """Average ms of one fn() call: a graph of `reps` back-to-back calls, events around it."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / reps)
    return best


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
    """A short eager sequence for counter collection: every (bits, M) GEMV of the step on
    four distinct weight copies, the prefill GEMM twice, decode attention over two copies of
    the 32K MHA quantized cache, and a 1 GiB copy twice (the copy is the calibration kernel:
    its bytes are known)."""
    dev = torch.device("cuda")
    K = N = 4096
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
    del hp, wt, xp, yp, wsp
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


def bench_moe(q, torch, workloads, stream, reps: int = 20):
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=32, help="rotating weight copies (>= 1 GB total)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=512 GEMM secondary line")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer decode stack line")
    ap.add_argument("--no-moe", action="store_true", help="skip the routed-expert FFN line")
    ap.add_argument("--no-kv", action="store_true", help="skip the quantized-KV decode attention line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="eager launches only (each GEMV of the step, the prefill GEMM, a 1 GiB copy) for "
                         "hardware-counter runs; prints no JSON")
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
    bits_list, m_list = workloads.SWEEP_BITS, workloads.SWEEP_M

    if args.pmc_pass:
        pmc_pass(q, torch, workloads)
        return

    log("bench: quantize + pack 4096x4096 at 2/3/5/6 bits")
    w = workloads.layer_weights(2)
    W = {}
    for b in bits_list:
        d, wt = quantize_pack(q, torch, w, b)
        copies = [dict(packed=wt["packed"].clone(), scales=wt["scales"].clone(), zeros=wt["zeros"].clone())
                  for _ in range(args.copies)]
        W[b] = (d, [q.weight(c["packed"], c["scales"], c["zeros"]) for c in copies], copies)
    X = {m: torch.from_numpy(workloads.activations_fp16(m, K, workloads.seed_for(2)).view(np.int16)).to(dev)
         for m in m_list}
    Y = {(b, m): torch.empty((m, N), dtype=torch.int16, device=dev) for b in bits_list for m in m_list}
    step_bytes = sum(weight_bytes(N, K, b) for b in bits_list) * len(m_list)
    total_copy_bytes = sum(weight_bytes(N, K, b) for b in bits_list) * args.copies
    log(f"bench: {args.copies} copies, {total_copy_bytes / 2**30:.2f} GiB of packed weights")

    def step(c):
        # every GEMV of a step reads its own weight copy, so no launch finds the previous
        # launch's bytes in the Infinity Cache
        for b in bits_list:
            d, hs, _ = W[b]
            for mi, m in enumerate(m_list):
                q.qlinear_gemv(d, hs[(c * len(m_list) + mi) % args.copies], X[m], K, m, Y[(b, m)], N)

    stream = torch.cuda.Stream()
    graphs = []
    for c in range(args.copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(c)
        graphs.append(g)
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup} steps")
    for i in range(args.warmup):
        graphs[i % args.copies].replay()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            graphs[i % args.copies].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    value = step_bytes * args.steps / (ms_total * 1e-3) / 1e9

    # per-kernel live timing (graphs of back-to-back launches of one (bits, M) kernel)
    log("bench: per-kernel timing")
    per = {}
    for b in bits_list:
        d, hs, _ = W[b]
        for m in m_list:
            fn = lambda i, d=d, hs=hs, m=m, b=b: q.qlinear_gemv(d, hs[i % args.copies], X[m], K, m, Y[(b, m)], N)
            ms = time_graph(torch, fn, 4 * args.copies, stream)
            per[f"b{b}_m{m}"] = dict(us=ms * 1e3, GBps=weight_bytes(N, K, b) / (ms * 1e-3) / 1e9)
    dom = max(per, key=lambda key: per[key]["us"])
    b_dom = int(dom.split("_")[0][1:])
    dom_bytes = weight_bytes(N, K, b_dom)
    achieved = dom_bytes / (per[dom]["us"] * 1e-6) / 1e9
    kname = gemv_kernel_name(b_dom, int(dom.split("_m")[1]), N)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(kname),
                    kernel=f"{kname} ({dom})", bytes_per_launch=dom_bytes,
                    avg_launch_us=round(per[dom]["us"], 3))

    extra = {}
    if not args.no_prefill:
        log("bench: prefill GEMM M=512 K=8192 N=28672 4-bit + 0.1% outliers")
        wp, _ = workloads.prefill_weights()
        dp, wt = quantize_pack(q, torch, wp, 4, workloads.PREFILL_OUTLIER_FRAC)
        del wp
        hp = q.weight(wt["packed"], wt["scales"], wt["zeros"], wt["rowptr"], wt["col"], wt["val"], wt["nnz"])
        xp = torch.from_numpy(workloads.prefill_activations().view(np.int16)).to(dev)
        Mp, Kp, Np = workloads.PREFILL_M, workloads.PREFILL_K, workloads.PREFILL_N
        yp = torch.empty((Mp, Np), dtype=torch.int16, device=dev)
        wsb = q.qlinear_gemm_workspace_bytes(dp, Mp, wt["nnz"])
        wsp = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda i: q.qlinear_gemm(dp, hp, xp, Kp, Mp, yp, Np, wsp, wsb), 10, stream)
        flops = 2 * Mp * Np * Kp + 2 * Mp * wt["nnz"]
        tf = flops / (ms * 1e-3) / 1e12
        extra["prefill_gemm_m512"] = dict(us=round(ms * 1e3, 2), TFLOPs=round(tf, 1),
                                          frac_mfma_f16=round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                          flops=flops, kernel="qp::gemm_kernel<4>")
        del hp, wt, xp, yp

    log("bench: 4096x4096 4-bit GEMV at M=1")
    d4, w4 = quantize_pack(q, torch, workloads.layer_weights(1), 4)
    c4 = [clone_weight(torch, w4) for _ in range(args.copies)]
    h4 = [q.weight(c["packed"], c["scales"], c["zeros"]) for c in c4]
    x1 = torch.from_numpy(workloads.activations_fp16(1, K, workloads.seed_for(1)).view(np.int16)).to(dev)
    y1 = torch.empty((1, N), dtype=torch.int16, device=dev)
    ms4 = time_graph(torch, lambda i: q.qlinear_gemv(d4, h4[i % args.copies], x1, K, 1, y1, N), 4 * args.copies,
                     stream)
    b4 = weight_bytes(N, K, 4)
    extra["gemv_4096_4bit_m1"] = dict(us=round(ms4 * 1e3, 3), GBps=round(b4 / (ms4 * 1e-3) / 1e9, 1),
                                      frac_hbm_peak=round(b4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      kernel=gemv_kernel_name(4, 1, N))
    del c4, h4, w4
    log("bench: 4096x4096 symmetric 2- and 3-bit GEMV at M=1 (no zero points)")
    sym = {}
    for b in (2, 3):
        ds, wsy = quantize_pack(q, torch, workloads.layer_weights(2), b, sym=True)
        cs = [clone_weight(torch, wsy) for _ in range(args.copies)]
        hs = [q.weight(c["packed"], c["scales"], None) for c in cs]
        ms = time_graph(torch, lambda i: q.qlinear_gemv(ds, hs[i % args.copies], x1, K, 1, y1, N), 4 * args.copies,
                        stream)
        bs = weight_bytes(N, K, b, sym=True)
        sym[f"b{b}_m1"] = dict(us=round(ms * 1e3, 3), GBps=round(bs / (ms * 1e-3) / 1e9, 1), bytes=bs)
        del cs, hs, wsy
    extra["gemv_4096_sym_m1"] = sym
    log("bench: 4096x4096 GEMV at M=1 with groups of 32 and 64")
    small = {}
    for b, g, sy in ((2, 32, True), (2, 64, True), (2, 32, False), (5, 64, False), (6, 64, False)):
        ds, wsy = quantize_pack(q, torch, workloads.layer_weights(2), b, sym=sy, g=g)
        cs = [clone_weight(torch, wsy) for _ in range(args.copies)]
        hs = [q.weight(c["packed"], c["scales"], c["zeros"]) for c in cs]
        ms = time_graph(torch, lambda i: q.qlinear_gemv(ds, hs[i % args.copies], x1, K, 1, y1, N), 4 * args.copies,
                        stream)
        bs = weight_bytes(N, K, b, sym=sy, g=g)
        small[f"b{b}_g{g}{'_sym' if sy else ''}"] = dict(us=round(ms * 1e3, 3), GBps=round(bs / (ms * 1e-3) / 1e9, 1),
                                                         bytes=bs, bits_per_weight=round(8 * bs / (N * K), 4))
        del cs, hs, wsy
    extra["gemv_4096_small_groups_m1"] = small
    log("bench: 4096x4096 GEMV at M=1 with zero points in b bits")
    pz = {}
    for b, g in ((2, 32), (3, 64), (5, 64), (6, 128)):
        dz = q.desc(b, N, K, group_size=g, zero_mode=q.QP_ZERO_PACKED)
        _, wz = quantize_pack(q, torch, workloads.layer_weights(2), b, g=g)
        zp = torch.empty(q.qp_zero_bytes(dz), dtype=torch.uint8, device=dev)
        q.qpack_pack_zeros(dz, wz["zeros"], zp)
        cs = [dict(packed=wz["packed"].clone(), scales=wz["scales"].clone(), zeros=zp.clone())
              for _ in range(args.copies)]
        hs = [q.weight(c["packed"], c["scales"], c["zeros"]) for c in cs]
        ms = time_graph(torch, lambda i: q.qlinear_gemv(dz, hs[i % args.copies], x1, K, 1, y1, N), 4 * args.copies,
                        stream)
        bz = N * K * b // 8 + (N * K // g) * 2 + q.qp_zero_bytes(dz)
        pz[f"b{b}_g{g}"] = dict(us=round(ms * 1e3, 3), GBps=round(bz / (ms * 1e-3) / 1e9, 1), bytes=bz,
                                bits_per_weight=round(8 * bz / (N * K), 4))
        del cs, hs, wz, zp
    extra["gemv_4096_packed_zeros_m1"] = pz
    if not args.no_stack:
        log("bench: Llama-7B-shaped 32-layer decode stack at M=1")
        extra["stack_llama7b_m1"] = bench_stack(q, torch, workloads, stream)
    if not args.no_moe:
        log("bench: routed-expert FFN, 16 experts, 128 tokens top-2")
        extra["moe_16x_ffn_t128"] = bench_moe(q, torch, workloads, stream)
    if not args.no_kv:
        log("bench: decode attention over an INT4-K / INT8-V cache (32K MHA, 4 x 8K GQA)")
        extra["kv_decode_attention"] = bench_kv(q, torch, workloads, stream)

    log("bench: 1 GiB device copy")
    extra["copy_GBps"] = round(copy_gbps(torch), 1)

    cpu = cpu1 = None
    if not args.no_cpu:
        import oracle
        log("bench: CPU oracle baseline")
        refs = {b: oracle.quantize(w, b) for b in bits_list}
        xs = {m: workloads.activations_fp16(m, K, workloads.seed_for(2)) for m in m_list}
        t0 = time.perf_counter()
        reps = 0
        while True:
            for b in bits_list:
                for m in m_list:
                    oracle.linear(xs[m], refs[b])
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 50:
                break
        dt = time.perf_counter() - t0
        cpu = dict(value=round(step_bytes * reps / dt / 1e9, 4), unit="GB/s", cores=oracle.num_threads(),
                   kind="oracle",
                   sample=f"{reps} full steps (12 fp64 GEMVs over the oracle's own codes), {dt:.1f} s")
        # the same oracle on one thread, over one step
        threads = oracle.num_threads()
        oracle.set_num_threads(1)
        t0 = time.perf_counter()
        for b in bits_list:
            for m in m_list:
                oracle.linear(xs[m], refs[b])
        dt1 = time.perf_counter() - t0
        oracle.set_num_threads(threads)
        cpu1 = dict(value=round(step_bytes / dt1 / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                    sample=f"1 full step (12 fp64 GEMVs over the oracle's own codes) on one thread, {dt1:.1f} s")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "4096x4096 layer, bits {2,3,5,6} x decode M {1,4,8}, asymmetric g=128, "
                               "page units, device tile layout",
                   "bits": list(bits_list), "m": list(m_list), "n": N, "k": K,
                   "weight_copies": args.copies, "step_weight_bytes": step_bytes,
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "per_kernel": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in per.items()},
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
