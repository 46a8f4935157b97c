"""Seeded synthetic inputs shaped like the workloads on the weight-only mixed-bit pages.

This module only draws random numbers and arranges them into arrays.  It holds none of
the quantization, packing or matmul arithmetic: both the CPU oracle and the GPU library
receive these arrays as inputs, so the two sides never share method code.

Recipe (numpy PCG64 via ``numpy.random.default_rng``):
  * weights  ~ N(0, 0.02): float32 draws scaled by 0.02, rounded RNE to fp16;
  * activations ~ N(0, 1): float32 draws rounded RNE to fp16;
  * planted outliers: floor(frac*N*K) positions uniform without replacement,
    magnitude U[3, 5], random sign (the bulk-vs-outlier picture of the 70B page,
    section 2: most weights in [-0.5, 0.5], a few with |w| > 3);
  * MoE routing: expert popularity p_r proportional to r^-s (Zipf), router logits
    log(p) + Gumbel(0, 1) per token, top-k by logit, combine weights = softmax of the
    logits taken at the chosen experts (not renormalised).
  * KV cache: K and V head vectors (head_dim 128) ~ N(0, 1) rounded to fp16 -- the KV page
    (s1.2) describes projected K/V as concentrated without extreme outliers; queries ~ N(0, 1);
    sequence lengths uniform in [lo, hi] for ragged batches.
Seeds: 1000*w + 16*layer + matrix_index, where w numbers the seed stream of a workload:
1 the 4096 x 4096 layer at 4 bits, 2 the same layer swept over 2/3/5/6 bits and M = 1/4/8,
3 the 32-layer Llama-7B-shaped stack, 4 the M = 512 prefill GEMM, 5 the 16-expert FFN, 6 the
quantized KV cache (matrix 0 = K, 1 = V; queries and lengths use the activation offset).
Activations use seed + 500000.
"""
from __future__ import annotations

import math

import numpy as np

ACT_SEED_OFFSET = 500_000
LLAMA_MATRICES = ("q", "k", "v", "o", "gate", "up", "down")


def seed_for(stream: int, layer: int = 0, matrix: int = 0) -> int:
    return 1000 * stream + 16 * layer + matrix


def normal_fp16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """fp16 array of N(0, std^2) draws (float32 draw * std, then RNE to fp16)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.astype(np.float16)


def weights_fp16(n: int, k: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Weight matrix W[n, k] (output features x input features), fp16."""
    return normal_fp16((n, k), seed, std)


def activations_fp16(m: int, k: int, seed: int) -> np.ndarray:
    """Activation rows x[m, k] ~ N(0, 1), fp16."""
    return normal_fp16((m, k), seed + ACT_SEED_OFFSET, 1.0)


def outlier_count(n: int, k: int, frac: float) -> int:
    return int(math.floor(frac * float(n * k)))


def plant_outliers(w: np.ndarray, frac: float, seed: int, lo: float = 3.0, hi: float = 5.0):
    """Overwrite floor(frac*N*K) uniformly chosen entries of ``w`` (in place) with
    values of magnitude U[lo, hi] and random sign.  Returns the sorted flat positions."""
    n, k = w.shape
    cnt = outlier_count(n, k, frac)
    rng = np.random.default_rng(seed + 7_000_000)
    pos = np.sort(rng.choice(n * k, size=cnt, replace=False))
    mag = rng.uniform(lo, hi, size=cnt).astype(np.float32)
    sign = np.where(rng.integers(0, 2, size=cnt) == 1, np.float32(1), np.float32(-1))
    w.reshape(-1)[pos] = (mag * sign).astype(np.float16)
    return pos


def zipf_routing(tokens: int, experts: int, topk: int, s: float, seed: int):
    """Top-k expert choice per token with Zipf(s)-skewed popularity.

    Returns (ids int32 [T, topk], weights float32 [T, topk]).  Expert e has popularity
    rank e+1.  The combine weight of a chosen expert is its softmax probability over all
    router logits (the top-k entries are not renormalised)."""
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    logp = -s * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    gumbel = rng.gumbel(size=(tokens, experts))
    logits = logp[None, :] + gumbel
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    z = logits - logits.max(axis=1, keepdims=True)
    prob = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    wts = np.take_along_axis(prob, order, axis=1).astype(np.float32)
    return order.astype(np.int32), wts


def interleave_row_blocks(a: np.ndarray, b: np.ndarray, block: int = 16) -> np.ndarray:
    """Rows of ``a`` and ``b`` interleaved in blocks of ``block`` rows:
    [a[0:16], b[0:16], a[16:32], b[16:32], ...].  Used to lay gate and up projections
    side by side so one pass over the pair can apply the SwiGLU epilogue."""
    assert a.shape == b.shape and a.shape[0] % block == 0
    n, k = a.shape
    out = np.empty((2 * n, k), dtype=a.dtype)
    out.reshape(n // block, 2, block, k)[:, 0] = a.reshape(n // block, block, k)
    out.reshape(n // block, 2, block, k)[:, 1] = b.reshape(n // block, block, k)
    return out


# ---------------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------------

# Single 4096x4096 layer (seed streams 1 and 2).
LAYER_N = 4096
LAYER_K = 4096
SWEEP_BITS = (2, 3, 5, 6)
SWEEP_M = (1, 4, 8)

# Llama-7B-shaped decode stack (seed stream 3).
STACK_LAYERS = 32
STACK_SHAPES = {  # (N, K) per matrix
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}

# Prefill-shaped dequant-GEMM with outliers (seed stream 4).
PREFILL_M, PREFILL_K, PREFILL_N = 512, 8192, 28672
PREFILL_OUTLIER_FRAC = 0.001

# MoE grouped experts (seed stream 5).
MOE_EXPERTS, MOE_DMODEL, MOE_DFF, MOE_TOKENS, MOE_TOPK, MOE_ZIPF = 16, 4096, 14336, 128, 2, 1.1


# Quantized KV-cache decode (seed stream 6): the KV page's 7B MHA layer (32 heads x 128) at a 32K
# context, and a GQA layer (8 KV heads, 8 query heads each) with four sequences of 8K.
KV_HEAD_DIM = 128
KV_MHA = dict(batch=1, q_heads=32, kv_heads=32, capacity=32768)
KV_GQA = dict(batch=4, q_heads=64, kv_heads=8, capacity=8192)


def kv_rows(rows: int, seed: int) -> np.ndarray:
    """rows head vectors [rows, 128] ~ N(0, 1), fp16 (K or V of cache rows 0 .. rows-1)."""
    return normal_fp16((rows, KV_HEAD_DIM), seed)


def kv_queries(batch: int, q_heads: int, seed: int) -> np.ndarray:
    return normal_fp16((batch, q_heads, KV_HEAD_DIM), seed + ACT_SEED_OFFSET)


def kv_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Ragged sequence lengths, uniform integers in [lo, hi]."""
    rng = np.random.default_rng(seed + ACT_SEED_OFFSET + 1)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def stack_bits(layer: int, name: str) -> int:
    """Bit width per matrix of the 32-layer stack.  The mixed table of the mixed-bit
    page (section 2.2) gives shares by bit width rather than a per-matrix table; this
    assignment follows its placement rules (first/last layers 6-bit, value and
    residual-end projections wide, middle FFN gate/up at 2 bits, a few 3-bit layers
    near the output) and averages 3.467 bits per weight over the Llama-7B shapes."""
    if layer == 0 or layer == STACK_LAYERS - 1:
        return 6
    table = {"gate": 2, "up": 2, "v": 6, "o": 5, "down": 5}
    if name in table:
        return table[name]
    return 2 if layer <= 21 else 3  # q and k


def stack_matrix_seed(layer: int, name: str) -> int:
    return seed_for(3, layer, LLAMA_MATRICES.index(name))


def layer_weights(stream: int = 1) -> np.ndarray:
    """The single 4096x4096 layer (seed stream 1: the 4-bit layer, 2: the bit sweep)."""
    return weights_fp16(LAYER_N, LAYER_K, seed_for(stream))


def prefill_weights() -> tuple[np.ndarray, np.ndarray]:
    """Configuration 4: W[28672, 8192] ~ N(0, 0.02) with 0.1% planted outliers.
    Returns (W, sorted flat positions of the planted outliers)."""
    w = weights_fp16(PREFILL_N, PREFILL_K, seed_for(4))
    pos = plant_outliers(w, PREFILL_OUTLIER_FRAC, seed_for(4))
    return w, pos


def prefill_activations() -> np.ndarray:
    return activations_fp16(PREFILL_M, PREFILL_K, seed_for(4))


def moe_expert(e: int, d_model: int = MOE_DMODEL, d_ff: int = MOE_DFF, stream: int = 5):
    """(gate [d_ff, d_model], up [d_ff, d_model], down [d_model, d_ff]) of expert e."""
    g = weights_fp16(d_ff, d_model, seed_for(stream, e, LLAMA_MATRICES.index("gate")))
    u = weights_fp16(d_ff, d_model, seed_for(stream, e, LLAMA_MATRICES.index("up")))
    d = weights_fp16(d_model, d_ff, seed_for(stream, e, LLAMA_MATRICES.index("down")))
    return g, u, d


def moe_inputs(tokens: int = MOE_TOKENS, d_model: int = MOE_DMODEL, experts: int = MOE_EXPERTS,
               topk: int = MOE_TOPK, stream: int = 5):
    """(x [tokens, d_model] fp16, ids int32 [tokens, topk], weights float32 [tokens, topk])."""
    x = activations_fp16(tokens, d_model, seed_for(stream))
    ids, wts = zipf_routing(tokens, experts, topk, MOE_ZIPF, seed_for(stream) + 900_000)
    return x, ids, wts
