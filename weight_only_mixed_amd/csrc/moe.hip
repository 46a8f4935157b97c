// Routed-expert plumbing: sort the tokens' top-k choices by expert and combine the expert
// outputs per token (on-device MoE page, s4.2: each expert task carries the hidden states of
// the tokens routed to it and their top-k expert ids; results return per token).
//
// Dispatch is one workgroup: expert sizes by LDS atomics, an exclusive scan for the offsets,
// then a stable placement (token order, then choice order) over chunks of 1024 choices: a
// choice's rank is its position among its wave's choices of the same expert (one ballot per
// expert) plus the counts of the chunk's earlier waves and of the earlier chunks.  Combine sums a token's choices in choice order in fp32 (no atomics),
// so results are deterministic.
#include "qp_internal.h"

namespace qp {

__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t *ids, const float *w,
                                                        int total, int topk, int n_experts,
                                                        int32_t *offsets, int32_t *row_src,
                                                        float *row_weight, int32_t *token_rows)
{
    __shared__ int cnt[kMaxExperts], base[kMaxExperts + 1], run[kMaxExperts];
    __shared__ int wcnt[16][kMaxExperts];  // per-wave counts of the current chunk
    const int t = threadIdx.x;
    if (t < kMaxExperts) cnt[t] = 0;
    __syncthreads();
    for (int i = t; i < total; i += 1024) {
        const int e = ids[i];
        if (e >= 0 && e < n_experts) atomicAdd(&cnt[e], 1);  // out-of-range ids are dropped
    }
    __syncthreads();
    if (t == 0) {
        int a = 0;
        for (int e = 0; e < n_experts; ++e) {
            base[e] = a;
            run[e] = 0;
            a += cnt[e];
        }
        base[n_experts] = a;
    }
    __syncthreads();
    if (t <= n_experts) offsets[t] = base[t];
    const int lane = t & 63, wv = t >> 6;
    for (int c0 = 0; c0 < total; c0 += 1024) {
        const int i = c0 + t;
        const int e_i = i < total ? ids[i] : -1;
        const bool ok = e_i >= 0 && e_i < n_experts;
        // this choice's rank among the wave's choices of the same expert, and the wave's count
        // of each expert (one ballot per expert, no barrier)
        int rank = 0;
        for (int e = 0; e < n_experts; ++e) {
            const uint64_t mask = __ballot(ok && e_i == e);
            if (ok && e_i == e) rank = __popcll(mask & ((1ull << lane) - 1));
            if (lane == 0) wcnt[wv][e] = __popcll(mask);
        }
        __syncthreads();
        int pos = -1;
        if (ok) {  // after the expert's earlier chunks and this chunk's earlier waves
            int before = 0;
            for (int w2 = 0; w2 < wv; ++w2) before += wcnt[w2][e_i];
            pos = base[e_i] + run[e_i] + before + rank;
        }
        __syncthreads();
        if (t < n_experts) {
            int c = 0;
            for (int w2 = 0; w2 < 16; ++w2) c += wcnt[w2][t];
            run[t] += c;
        }
        __syncthreads();
        if (i < total) {
            if (pos < 0) {
                token_rows[i] = -1;
            } else {
                row_src[pos] = i / topk;
                row_weight[pos] = w[i];
                token_rows[i] = pos;
            }
        }
    }
}

__global__ __launch_bounds__(256) void combine_kernel(const float *rows, int64_t ld_rows,
                                                      const int32_t *token_rows,
                                                      const float *row_weight, int topk,
                                                      int64_t n, uint16_t *out, int64_t ldo,
                                                      int nsplit, int64_t split_stride)
{
    const int64_t tok = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n) return;
    float s = 0.0f;
    for (int j = 0; j < topk; ++j) {
        const int32_t r = token_rows[tok * topk + j];
        if (r < 0) continue;
        // a row computed in k parts: its partial rows summed in part order first
        float v = rows[r * ld_rows + c];
        for (int p = 1; p < nsplit; ++p) v += rows[p * split_stride + r * ld_rows + c];
        s = __builtin_fmaf(row_weight[r], v, s);
    }
    out[tok * ldo + c] = __builtin_bit_cast(uint16_t, (_Float16)s);
}

hipError_t launch_moe_dispatch(const int32_t *ids, const float *w, int64_t tokens, int topk,
                               int n_experts, int32_t *offsets, int32_t *row_src,
                               float *row_weight, int32_t *token_rows, hipStream_t st)
{
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(1024), 0, st, ids, w, (int)(tokens * topk),
                       topk, n_experts, offsets, row_src, row_weight, token_rows);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float *rows, int64_t ld_rows, const int32_t *token_rows,
                              const float *row_weight, int64_t tokens, int topk, int64_t n,
                              uint16_t *out, int64_t ldo, int nsplit, int64_t split_stride,
                              hipStream_t st)
{
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)tokens), dim3(256),
                       0, st, rows, ld_rows, token_rows, row_weight, topk, n, out, ldo, nsplit, split_stride);
    return hipGetLastError();
}

}  // namespace qp
