// Dynamic per-token int8 activations for the integer-dot path (inference acceleration guide,
// s1.2: W8A8 quantizes activations to INT8 dynamically, per token, so the matrix product runs on
// the integer matrix units).  Row m: a = max |x|, s = a / 127, xq = clamp(rint(x / s), -127,
// 127) in IEEE fp32 (compiled without contraction; correctly rounded division, round half to
// even), all-zero rows s = 0 and xq = 0.  The codes go to the int8 storage map of qpack.h: in
// each 128-k group, 16-byte piece 4s + t holds k = 64s + 8t .. +7 then 64s + 32 + 8t .. +7.
#include "qp_internal.h"

namespace qp {

namespace {

__device__ __forceinline__ float hf(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Storage position of the 8-k block starting at k0 (k0 % 8 == 0) inside its row.
__device__ __forceinline__ int64_t act_block_pos(int64_t k0)
{
    const int64_t g = k0 >> 7, kk = k0 & 127, st = kk >> 6, rem = kk & 63;
    return g * 128 + 16 * (4 * st + ((rem & 31) >> 3)) + 8 * (rem >> 5);
}

// One workgroup per row: the row's maximum |x| (waves shuffle, then LDS), then every thread
// quantizes 8-k blocks and stores each as 8 bytes at its storage position.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t *x, int64_t ldx, int64_t k, int8_t *xq,
                                                        float *scales)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * ldx;
    const int tid = threadIdx.x;
    float a = 0.f;
    for (int64_t k0 = 8 * (int64_t)tid; k0 < k; k0 += 8 * 256) {
        const u4 v = *(const u4 *)(xr + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a = fmaxf(a, fabsf(hf((uint16_t)(v[e] & 0xFFFF))));
            a = fmaxf(a, fabsf(hf((uint16_t)(v[e] >> 16))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __fdiv_rn(a, 127.0f);
    if (tid == 0) scales[row] = a == 0.f ? 0.f : s;
    int8_t *dst = xq + row * k;
    for (int64_t k0 = 8 * (int64_t)tid; k0 < k; k0 += 8 * 256) {
        const u4 v = *(const u4 *)(xr + k0);
        uint32_t out[2] = {0u, 0u};
        if (a != 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = hf((uint16_t)(v[e / 2] >> (16 * (e & 1))));
                const float q = fminf(fmaxf(rintf(__fdiv_rn(xv, s)), -127.f), 127.f);
                out[e / 4] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (e & 3));
            }
        }
        *(u2 *)(dst + act_block_pos(k0)) = (u2){out[0], out[1]};
    }
}

}  // namespace

hipError_t launch_act_quantize(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int8_t *xq, float *scales,
                               hipStream_t st)
{
    hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)m), dim3(256), 0, st, x, ldx, k, xq, scales);
    return hipGetLastError();
}

}  // namespace qp
