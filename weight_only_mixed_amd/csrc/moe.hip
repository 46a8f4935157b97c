// Routed-expert plumbing: sort the tokens' top-k choices by expert and combine the expert
// outputs per token (on-device MoE page, s4.2: each expert task carries the hidden states of
// the tokens routed to it and their top-k expert ids; results return per token).
//
// Dispatch is one workgroup: expert sizes by LDS atomics, an exclusive scan for the offsets,
// then a stable placement (token order, then choice order) by one block scan per expert over
// chunks of 1024 choices.  Combine sums a token's choices in choice order in fp32 (no atomics),
// so results are deterministic.
#include "qp_internal.h"

namespace qp {

__device__ int block_excl_scan_1024(int v, int *lds, int *total)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[wv] = x;
    __syncthreads();
    if (t == 0) {
        int a = 0;
        for (int i = 0; i < 16; ++i) {
            const int c = lds[i];
            lds[i] = a;
            a += c;
        }
        lds[16] = a;
    }
    __syncthreads();
    const int res = lds[wv] + x - v;
    *total = lds[16];
    __syncthreads();
    return res;
}

__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t *ids, const float *w,
                                                        int total, int topk, int n_experts,
                                                        int32_t *offsets, int32_t *row_src,
                                                        float *row_weight, int32_t *token_rows)
{
    __shared__ int cnt[kMaxExperts], base[kMaxExperts + 1], run[kMaxExperts];
    __shared__ int lds[17];
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
    for (int c0 = 0; c0 < total; c0 += 1024) {
        const int i = c0 + t;
        const int e_i = i < total ? ids[i] : -1;
        int pos = -1;
        for (int e = 0; e < n_experts; ++e) {
            int tot;
            const int rk = block_excl_scan_1024(e_i == e ? 1 : 0, lds, &tot);
            if (e_i == e) pos = base[e] + run[e] + rk;
            __syncthreads();
            if (t == 0) run[e] += tot;
            __syncthreads();
        }
        if (i < total && pos < 0) token_rows[i] = -1;
        if (i < total && pos >= 0) {
            row_src[pos] = i / topk;
            row_weight[pos] = w[i];
            token_rows[i] = pos;
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
