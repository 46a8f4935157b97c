// Group quantizer with fp8 scales and an fp16 fallback (mixed-bit page, s2.3: 8-bit float
// scales, the few blocks out of the fp8 range kept in fp16).  One workgroup per row, three
// passes over the row (each wave takes 128-value chunks, two values per lane, a group's lanes
// reducing its range with shuffles, as the fp16 quantizer does):
//  1. every group's fp32 scale s32 (the fp16 quantizer's, before its fp16 rounding) and the
//     row's largest: factor F = max * 2^-8 (exact; that group maps to 256);
//  2. which groups fall below E4M3's normal range (s32 / F < 2^-6): flags in LDS, ranked in
//     group order by a workgroup scan, counted into counts[row];
//  3. per group the scale byte (the smallest E4M3 value >= s32 / F, or 0x80 | rank with the
//     fp16 scale in the row's fallback list, or 0 for an all-zero group), the zero point and
//     the codes, all from the stored scale.
// IEEE fp32 with explicit round-to-nearest operations (compiled without contraction), so the
// result is bit-identical to the CPU reference.
#include "qp_internal.h"

namespace qp {

namespace {

constexpr int kChunk = 128;         // values of a row one wave handles at a time
constexpr int kMaxGroupsLds = 16384;  // groups per row the LDS flag and rank arrays hold

// Range of the group holding this lane's two values (lanes [j gs/2, (j+1) gs/2) hold group j):
// lo = min(min w, 0), hi = max(max w, 0), m = max |w|.
__device__ __forceinline__ void group_range(float v0, float v1, int gs, float &lo, float &hi, float &m)
{
    lo = fminf(fminf(v0, v1), 0.0f);
    hi = fmaxf(fmaxf(v0, v1), 0.0f);
    m = fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
    for (int off = gs / 4; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off));
        hi = fmaxf(hi, __shfl_xor(hi, off));
        m = fmaxf(m, __shfl_xor(m, off));
    }
}

// fp32 scale of a group (valid when !zero): (hi - lo) / qmax, or (m + m) / qmax for symmetric.
template <int BITS, bool SYM>
__device__ __forceinline__ float group_s32(float lo, float hi, float m, bool &zero)
{
    constexpr int qmax = (1 << BITS) - 1;
    zero = SYM ? (m == 0.0f) : (hi == lo);
    return __fdiv_rn(SYM ? __fadd_rn(m, m) : __fsub_rn(hi, lo), (float)qmax);
}

// The smallest E4M3 code whose value is >= t, for t in [2^-6, 256] (a normal fp32): keep the
// exponent, round the mantissa up to 3 bits.
__device__ __forceinline__ uint32_t e4m3_ceil(float t)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, t);
    int e = (int)((b >> 23) & 0xFF) - 127;
    const uint32_t man = b & 0x7FFFFF;
    uint32_t m3 = (man >> 20) + ((man & 0xFFFFF) ? 1u : 0u);
    if (m3 == 8) {
        m3 = 0;
        ++e;
    }
    return ((uint32_t)(e + 7) << 3) | m3;
}
// Value of a positive normal E4M3 code.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    return __builtin_ldexpf(1.0f + (float)(c & 7) * 0.125f, (int)((c >> 3) & 15) - 7);
}

// Exclusive scan of one int per thread across the 256-thread workgroup; total via *sum.
__device__ __forceinline__ int block_scan_256(int v, int *lds4, int *sum)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) lds4[wv] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wv; ++i) base += lds4[i];
    *sum = lds4[0] + lds4[1] + lds4[2] + lds4[3];
    __syncthreads();
    return base + incl - v;
}

template <int BITS, bool SYM>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t *w, int64_t ldw, int64_t k, int gs,
                                                           uint8_t *codes, uint8_t *sc8, uint8_t *zeros, float *factors,
                                                           uint16_t *fb, int64_t fb_stride, int32_t *counts)
{
    constexpr int qmax = (1 << BITS) - 1, mid = 1 << (BITS - 1);
    __shared__ uint8_t flag[kMaxGroupsLds];
    __shared__ int16_t rank[kMaxGroupsLds];
    __shared__ float red[4];
    __shared__ int scan4[4];
    const int64_t r = blockIdx.x;
    const uint16_t *row = w + r * ldw;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t nch = k / kChunk, G = k / gs;
    const int per = kChunk / gs;  // groups per chunk
    auto load2 = [&](int64_t c, float &v0, float &v1) {
        const uint32_t p = *(const uint32_t *)(row + c * kChunk + 2 * lane);
        v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFF));
        v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
    };

    // 1. the row's largest group scale
    float mx = 0.0f;
    for (int64_t c = wv; c < nch; c += 4) {
        float v0, v1, lo, hi, m;
        load2(c, v0, v1);
        group_range(v0, v1, gs, lo, hi, m);
        bool zero;
        const float s32 = group_s32<BITS, SYM>(lo, hi, m, zero);
        if (!zero) mx = fmaxf(mx, s32);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red[wv] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float F = mx > 0.0f ? __fmul_rn(mx, 0.00390625f) : 1.0f;  // exact: times 2^-8
    if (threadIdx.x == 0) factors[r] = F;

    // 2. groups below E4M3's normal range, ranked in group order
    for (int64_t c = wv; c < nch; c += 4) {
        float v0, v1, lo, hi, m;
        load2(c, v0, v1);
        group_range(v0, v1, gs, lo, hi, m);
        bool zero;
        const float s32 = group_s32<BITS, SYM>(lo, hi, m, zero);
        if (lane % (gs / 2) == 0) flag[c * per + lane / (gs / 2)] = !zero && __fdiv_rn(s32, F) < 0.015625f;
    }
    __syncthreads();
    const int64_t span = (G + 255) / 256, g0 = threadIdx.x * span, g1 = min(G, g0 + span);
    int cnt = 0;
    for (int64_t gi = g0; gi < g1; ++gi) cnt += flag[gi];
    int total;
    int before = block_scan_256(cnt, scan4, &total);
    for (int64_t gi = g0; gi < g1; ++gi) {
        rank[gi] = (int16_t)before;
        before += flag[gi];
    }
    if (threadIdx.x == 0) counts[r] = total;
    __syncthreads();

    // 3. scale bytes, zero points and codes from the stored scales
    for (int64_t c = wv; c < nch; c += 4) {
        float v0, v1, lo, hi, m;
        load2(c, v0, v1);
        group_range(v0, v1, gs, lo, hi, m);
        bool zero;
        const float s32 = group_s32<BITS, SYM>(lo, hi, m, zero);
        const int64_t gi = c * per + lane / (gs / 2);
        const bool head = lane % (gs / 2) == 0;
        uint32_t q0, q1, byte;
        int zp = SYM ? mid : 0;
        if (zero) {
            byte = 0;
            q0 = q1 = (uint32_t)zp;
        } else {
            float sf;
            if (flag[gi]) {
                uint16_t sh = __builtin_bit_cast(uint16_t, (_Float16)s32);
                if ((sh & 0x7C00) == 0) sh = 0x0400;  // zero / subnormal -> 2^-14, as the fp16 path
                sf = (float)__builtin_bit_cast(_Float16, sh);
                const int j = rank[gi];
                byte = 0x80u | (uint32_t)(j & 0x7F);
                if (head && j < fb_stride) fb[r * fb_stride + j] = sh;
            } else {
                byte = e4m3_ceil(__fdiv_rn(s32, F));
                sf = __fmul_rn(F, e4m3_value(byte));
            }
            if constexpr (!SYM) {
                zp = -(int)__builtin_rintf(__fdiv_rn(lo, sf));
                zp = zp < 0 ? 0 : (zp > qmax ? qmax : zp);
            }
            const int a = (int)__builtin_rintf(__fdiv_rn(v0, sf)) + zp;
            const int b = (int)__builtin_rintf(__fdiv_rn(v1, sf)) + zp;
            q0 = a < 0 ? 0 : (a > qmax ? qmax : a);
            q1 = b < 0 ? 0 : (b > qmax ? qmax : b);
        }
        *(uint16_t *)(codes + r * k + c * kChunk + 2 * lane) = (uint16_t)(q0 | (q1 << 8));
        if (head) {
            sc8[r * G + gi] = (uint8_t)byte;
            if (zeros) zeros[r * G + gi] = (uint8_t)zp;
        }
    }
}

template <int BITS>
hipError_t launch_bits(bool sym, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs, uint8_t *codes,
                       uint8_t *sc8, uint8_t *zeros, float *factors, uint16_t *fb, int64_t fb_stride, int32_t *counts,
                       hipStream_t st)
{
    if (sym)
        hipLaunchKernelGGL((quantize_fp8_kernel<BITS, true>), dim3((unsigned)n), dim3(256), 0, st, w, ldw, k, gs, codes,
                           sc8, (uint8_t *)nullptr, factors, fb, fb_stride, counts);
    else
        hipLaunchKernelGGL((quantize_fp8_kernel<BITS, false>), dim3((unsigned)n), dim3(256), 0, st, w, ldw, k, gs,
                           codes, sc8, zeros, factors, fb, fb_stride, counts);
    return hipGetLastError();
}

}  // namespace

int64_t quantize_fp8_max_groups() { return kMaxGroupsLds; }

hipError_t launch_quantize_fp8(int bits, bool sym, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                               uint8_t *codes, uint8_t *sc8, uint8_t *zeros, float *factors, uint16_t *fb,
                               int64_t fb_stride, int32_t *counts, hipStream_t st)
{
    switch (bits) {
    case 2: return launch_bits<2>(sym, w, ldw, n, k, gs, codes, sc8, zeros, factors, fb, fb_stride, counts, st);
    case 3: return launch_bits<3>(sym, w, ldw, n, k, gs, codes, sc8, zeros, factors, fb, fb_stride, counts, st);
    case 4: return launch_bits<4>(sym, w, ldw, n, k, gs, codes, sc8, zeros, factors, fb, fb_stride, counts, st);
    case 5: return launch_bits<5>(sym, w, ldw, n, k, gs, codes, sc8, zeros, factors, fb, fb_stride, counts, st);
    case 6: return launch_bits<6>(sym, w, ldw, n, k, gs, codes, sc8, zeros, factors, fb, fb_stride, counts, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qp
