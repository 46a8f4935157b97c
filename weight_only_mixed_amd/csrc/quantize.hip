// Group quantizer and outlier hold-out on the GPU.
//
// Formula: inference-acceleration guide, s1.1 (scale = (max-min)/(qmax-qmin),
// zero_point = qmin - round(min/scale), q = round(x/scale) + zero_point).  Groups of 128
// along k and the top-0.1% |w| held out in fp16: single-GPU 70B page, s2.  fp16 scales:
// mixed-bit page, s2.3.  Arithmetic is IEEE fp32 with explicit round-to-nearest
// operations (this file is compiled without floating-point contraction), so the codes,
// scales and zero points are bit-identical to the CPU reference.
//
// Outlier selection is exact and deterministic: the k_out largest fp16 magnitudes, ties to
// the lower row-major index.  A 32768-bin histogram of magnitude bit patterns gives the
// threshold pattern T and how many of the elements equal to T are taken (need_eq); per-row
// counts and an ordered scan then assign every taken element its CSR slot.
#include "qp_internal.h"

namespace qp {

constexpr int kHistBins = 32768;

size_t quant_ws_bytes(int64_t n)
{
    return (size_t)kHistBins * 4 + 16 + 3 * (size_t)n * 4 + 256;
}

QuantWs quant_ws_carve(void *ws, int64_t n)
{
    uint8_t *p = (uint8_t *)ws;
    QuantWs q;
    q.hist = (uint32_t *)p;
    p += (size_t)kHistBins * 4;
    q.ctl = (uint32_t *)p;
    p += 16;
    q.gt_cnt = (int32_t *)p;
    p += (size_t)n * 4;
    q.eq_cnt = (int32_t *)p;
    p += (size_t)n * 4;
    q.eq_base = (int32_t *)p;
    return q;
}

__global__ void zero_u32_kernel(uint32_t *p, int64_t n)
{
    int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Histogram of fp16 magnitude patterns (w & 0x7FFF).  LDS-private, flushed with atomics.
__global__ __launch_bounds__(1024) void hist_kernel(const uint16_t *w, int64_t ldw, int64_t n,
                                                    int64_t k, uint32_t *hist)
{
    __shared__ uint32_t h[kHistBins];
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
        const uint32_t *row = (const uint32_t *)(w + r * ldw);
        for (int64_t c = threadIdx.x; c < k / 2; c += blockDim.x) {
            const uint32_t v = row[c];
            atomicAdd(&h[v & 0x7FFF], 1u);
            atomicAdd(&h[(v >> 16) & 0x7FFF], 1u);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
        if (h[i]) atomicAdd(&hist[i], h[i]);
}

// Threshold T: the largest magnitude pattern with count(mag >= T) >= kout.
// ctl[0] = T, ctl[1..2] = need_eq (int64) = kout - count(mag > T).
__global__ __launch_bounds__(1024) void threshold_kernel(const uint32_t *hist, int64_t kout,
                                                         uint32_t *ctl)
{
    __shared__ uint64_t part[1024];
    const int t = threadIdx.x;
    uint64_t s = 0;
    for (int i = 0; i < 32; ++i) s += hist[32 * t + i];
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        uint64_t acc = 0;
        for (int u = 1023; u >= 0; --u) {
            acc += part[u];
            part[u] = acc;  // elements with magnitude >= 32u
        }
    }
    __syncthreads();
    const uint64_t ge_here = part[t];
    const uint64_t ge_next = t < 1023 ? part[t + 1] : 0;
    if (ge_here >= (uint64_t)kout && ge_next < (uint64_t)kout) {
        uint64_t c = ge_next;
        for (int i = 31; i >= 0; --i) {
            const uint64_t before = c;
            c += hist[32 * t + i];
            if (c >= (uint64_t)kout) {
                const int64_t need = kout - (int64_t)before;
                ctl[0] = 32 * t + i;
                ctl[1] = (uint32_t)(need & 0xFFFFFFFF);
                ctl[2] = (uint32_t)((uint64_t)need >> 32);
                break;
            }
        }
    }
}

__device__ __forceinline__ int64_t need_eq_of(const uint32_t *ctl)
{
    return (int64_t)(((uint64_t)ctl[2] << 32) | ctl[1]);
}

// Per-row counts of magnitudes above and equal to T.
__global__ __launch_bounds__(256) void rowcount_kernel(const uint16_t *w, int64_t ldw, int64_t k,
                                                       const uint32_t *ctl, int32_t *gt_cnt,
                                                       int32_t *eq_cnt)
{
    __shared__ int sg[4], se[4];
    const uint32_t T = ctl[0];
    const uint16_t *row = w + blockIdx.x * ldw;
    int g = 0, e = 0;
    for (int64_t c = threadIdx.x; c < k; c += 256) {
        const uint32_t m = row[c] & 0x7FFF;
        g += m > T;
        e += m == T;
    }
    for (int off = 32; off > 0; off >>= 1) {
        g += __shfl_xor(g, off);
        e += __shfl_xor(e, off);
    }
    if ((threadIdx.x & 63) == 0) {
        sg[threadIdx.x >> 6] = g;
        se[threadIdx.x >> 6] = e;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        gt_cnt[blockIdx.x] = sg[0] + sg[1] + sg[2] + sg[3];
        eq_cnt[blockIdx.x] = se[0] + se[1] + se[2] + se[3];
    }
}

// Exclusive scan of a per-thread value across a 1024-thread block.
__device__ int64_t block_scan_excl_1024(int64_t v, int64_t *lds, int64_t *total)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int64_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[wv] = x;
    __syncthreads();
    if (t == 0) {
        int64_t a = 0;
        for (int i = 0; i < 16; ++i) {
            int64_t c = lds[i];
            lds[i] = a;
            a += c;
        }
        lds[16] = a;
    }
    __syncthreads();
    const int64_t res = lds[wv] + x - v;
    *total = lds[16];
    __syncthreads();
    return res;
}

// eq_base[r] = ties before row r; rowptr[r+1] = held-out count of rows 0..r.
__global__ __launch_bounds__(1024) void rowscan_kernel(int64_t n, const uint32_t *ctl,
                                                       const int32_t *gt_cnt,
                                                       const int32_t *eq_cnt, int32_t *eq_base,
                                                       int32_t *rowptr)
{
    __shared__ int64_t lds[17];
    const int64_t need = ctl ? need_eq_of(ctl) : 0;
    const int64_t per = (n + 1023) / 1024;
    const int64_t r0 = threadIdx.x * per, r1 = min(n, r0 + per);
    int64_t se = 0;
    for (int64_t r = r0; r < r1; ++r) se += ctl ? eq_cnt[r] : 0;
    int64_t tot;
    int64_t ebase = block_scan_excl_1024(se, lds, &tot);
    int64_t ss = 0;
    {
        int64_t eb = ebase;
        for (int64_t r = r0; r < r1; ++r) {
            const int64_t e = ctl ? eq_cnt[r] : 0;
            const int64_t take = min(max(need - eb, (int64_t)0), e);
            ss += (ctl ? gt_cnt[r] : 0) + take;
            eb += e;
        }
    }
    int64_t sbase = block_scan_excl_1024(ss, lds, &tot);
    if (threadIdx.x == 0) rowptr[0] = 0;
    int64_t eb = ebase, sb = sbase;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t e = ctl ? eq_cnt[r] : 0;
        const int64_t take = min(max(need - eb, (int64_t)0), e);
        if (eq_base) eq_base[r] = (int32_t)eb;
        sb += (ctl ? gt_cnt[r] : 0) + take;
        rowptr[r + 1] = (int32_t)sb;
        eb += e;
    }
}

// Exclusive scan across a 256-thread block (int).
__device__ int block_scan_excl_256(int v, int *lds)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[wv] = x;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wv; ++i) base += lds[i];
    __syncthreads();
    return base + x - v;
}

constexpr int kChunk = 128;  // weights of a row one wave quantizes at a time (groups of 32, 64 or 128)

// Quantize the symmetric groups of `gs` values (32, 64 or 128) in a wave's 128 values (two
// per lane, lanes [j gs/2, (j+1) gs/2) hold group j): range [-m, m] with m = max |w|, scale
// fp16((m + m) / qmax), codes around the implied midpoint 2^(b-1).  scale_out points at the
// chunk's first group.
template <int BITS>
__device__ __forceinline__ void quantize_group_wave_sym(float v0, float v1, int lane, int gs, uint8_t *codes_out,
                                                        uint16_t *scale_out)
{
    constexpr int qmax = (1 << BITS) - 1, z = 1 << (BITS - 1);
    float m = __builtin_fabsf(v0);
    if (__builtin_fabsf(v1) > m) m = __builtin_fabsf(v1);
    for (int off = gs / 4; off > 0; off >>= 1) {
        const float om = __shfl_xor(m, off);
        if (om > m) m = om;
    }
    uint16_t sbits;
    uint32_t q0, q1;
    if (m == 0.0f) {
        sbits = 0x3C00;  // 1.0
        q0 = q1 = z;
    } else {
        const float s32 = __fdiv_rn(__fadd_rn(m, m), (float)qmax);
        sbits = __builtin_bit_cast(uint16_t, (_Float16)s32);
        if ((sbits & 0x7C00) == 0) sbits = 0x0400;  // zero / subnormal -> 2^-14
        const float sf = (float)__builtin_bit_cast(_Float16, sbits);
        int a = (int)__builtin_rintf(__fdiv_rn(v0, sf)) + z;
        int b = (int)__builtin_rintf(__fdiv_rn(v1, sf)) + z;
        q0 = a < 0 ? 0 : (a > qmax ? qmax : a);
        q1 = b < 0 ? 0 : (b > qmax ? qmax : b);
    }
    *(uint16_t *)(codes_out + 2 * lane) = (uint16_t)(q0 | (q1 << 8));
    if (lane % (gs / 2) == 0) scale_out[lane / (gs / 2)] = sbits;
}

// Quantize the groups of `gs` values (32, 64 or 128) in a wave's 128 values: two values per
// lane, lanes [j gs/2, (j+1) gs/2) hold group j; scale_out / zero_out point at the chunk's
// first group.
template <int BITS>
__device__ __forceinline__ void quantize_group_wave(float v0, float v1, int lane, int gs,
                                                    uint8_t *codes_out, uint16_t *scale_out,
                                                    uint8_t *zero_out)
{
    constexpr int qmax = (1 << BITS) - 1;
    float lo = 0.0f, hi = 0.0f;
    if (v0 < lo) lo = v0;
    if (v0 > hi) hi = v0;
    if (v1 < lo) lo = v1;
    if (v1 > hi) hi = v1;
    for (int off = gs / 4; off > 0; off >>= 1) {
        const float olo = __shfl_xor(lo, off), ohi = __shfl_xor(hi, off);
        if (olo < lo) lo = olo;
        if (ohi > hi) hi = ohi;
    }
    uint16_t sbits;
    int zp;
    uint32_t q0, q1;
    if (hi == lo) {
        sbits = 0x3C00;  // 1.0
        zp = 0;
        q0 = q1 = 0;
    } else {
        const float range = __fsub_rn(hi, lo);
        const float s32 = __fdiv_rn(range, (float)qmax);
        sbits = __builtin_bit_cast(uint16_t, (_Float16)s32);
        if ((sbits & 0x7C00) == 0) sbits = 0x0400;  // zero / subnormal -> 2^-14
        const float sf = (float)__builtin_bit_cast(_Float16, sbits);
        zp = -(int)__builtin_rintf(__fdiv_rn(lo, sf));
        zp = zp < 0 ? 0 : (zp > qmax ? qmax : zp);
        int a = (int)__builtin_rintf(__fdiv_rn(v0, sf)) + zp;
        int b = (int)__builtin_rintf(__fdiv_rn(v1, sf)) + zp;
        q0 = a < 0 ? 0 : (a > qmax ? qmax : a);
        q1 = b < 0 ? 0 : (b > qmax ? qmax : b);
    }
    *(uint16_t *)(codes_out + 2 * lane) = (uint16_t)(q0 | (q1 << 8));
    if (lane % (gs / 2) == 0) {
        scale_out[lane / (gs / 2)] = sbits;
        zero_out[lane / (gs / 2)] = (uint8_t)zp;
    }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// One block per row.  With outliers: mark held-out elements in LDS (ordered scan), write
// their CSR entries, then quantize each group with held-out slots read as +0.  SYM: symmetric
// groups, no zero points written.
template <int BITS, bool OUTL, bool SYM>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const uint16_t *w, int64_t ldw, int64_t k, const uint32_t *ctl, const int32_t *eq_base,
    const int32_t *rowptr, uint8_t *codes, uint16_t *scales, uint8_t *zeros, int32_t *col,
    uint16_t *val, int gs)
{
    extern __shared__ uint8_t held[];  // k bytes (OUTL only)
    __shared__ int scan_lds[4];
    const int64_t r = blockIdx.x;
    const uint16_t *row = w + r * ldw;
    const int t = threadIdx.x;
    const int64_t G = k / gs, per = kChunk / gs;  // groups per row, per 128-value chunk

    if constexpr (OUTL) {
        const uint32_t T = ctl[0];
        const int64_t need = need_eq_of(ctl);
        const int64_t per = (k + 255) / 256;
        const int64_t c0 = t * per, c1 = min(k, c0 + per);
        int eqn = 0;
        for (int64_t c = c0; c < c1; ++c) eqn += (row[c] & 0x7FFF) == T;
        const int eq_before = block_scan_excl_256(eqn, scan_lds);
        int64_t rank = (int64_t)eq_base[r] + eq_before;
        int seln = 0;
        for (int64_t c = c0; c < c1; ++c) {
            const uint32_t m = row[c] & 0x7FFF;
            uint8_t h = 0;
            if (m > T) {
                h = 1;
            } else if (m == T) {
                h = rank < need;
                ++rank;
            }
            held[c] = h;
            seln += h;
        }
        const int sel_before = block_scan_excl_256(seln, scan_lds);
        int64_t pos = (int64_t)rowptr[r] + sel_before;
        for (int64_t c = c0; c < c1; ++c) {
            if (held[c]) {
                col[pos] = (int32_t)c;
                val[pos] = row[c];
                ++pos;
            }
        }
        __syncthreads();
    }

    const int lane = t & 63, wv = t >> 6;
    for (int64_t ch = wv; ch < k / kChunk; ch += 4) {
        const int64_t c = ch * kChunk + 2 * lane;
        const uint32_t pair = *(const uint32_t *)(row + c);
        float v0 = half_bits_to_float(pair & 0xFFFF), v1 = half_bits_to_float(pair >> 16);
        if constexpr (OUTL) {
            if (held[c]) v0 = 0.0f;
            if (held[c + 1]) v1 = 0.0f;
        }
        if constexpr (SYM)
            quantize_group_wave_sym<BITS>(v0, v1, lane, gs, codes + r * k + ch * kChunk, scales + r * G + ch * per);
        else
            quantize_group_wave<BITS>(v0, v1, lane, gs, codes + r * k + ch * kChunk, scales + r * G + ch * per,
                                      zeros + r * G + ch * per);
    }
}

template <int BITS, bool SYM>
static hipError_t quantize_bits(const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                                int64_t kout, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                                int32_t *rowptr, int32_t *col, uint16_t *val, const QuantWs &ws,
                                hipStream_t st)
{
    if (kout > 0) {
        hipLaunchKernelGGL(zero_u32_kernel, dim3((kHistBins + 255) / 256), dim3(256), 0, st,
                           ws.hist, (int64_t)kHistBins);
        const int nb = (int)(n < 1024 ? n : 1024);
        hipLaunchKernelGGL(hist_kernel, dim3(nb), dim3(1024), 0, st, w, ldw, n, k, ws.hist);
        hipLaunchKernelGGL(threshold_kernel, dim3(1), dim3(1024), 0, st, ws.hist, kout, ws.ctl);
        hipLaunchKernelGGL(rowcount_kernel, dim3(n), dim3(256), 0, st, w, ldw, k, ws.ctl,
                           ws.gt_cnt, ws.eq_cnt);
        hipLaunchKernelGGL(rowscan_kernel, dim3(1), dim3(1024), 0, st, n, ws.ctl, ws.gt_cnt,
                           ws.eq_cnt, ws.eq_base, rowptr);
        hipLaunchKernelGGL((quantize_rows_kernel<BITS, true, SYM>), dim3(n), dim3(256), (size_t)k, st,
                           w, ldw, k, ws.ctl, ws.eq_base, rowptr, codes, scales, zeros, col, val, gs);
    } else {
        if (rowptr)
            hipLaunchKernelGGL(rowscan_kernel, dim3(1), dim3(1024), 0, st, n,
                               (const uint32_t *)nullptr, (const int32_t *)nullptr,
                               (const int32_t *)nullptr, (int32_t *)nullptr, rowptr);
        hipLaunchKernelGGL((quantize_rows_kernel<BITS, false, SYM>), dim3(n), dim3(256), 0, st, w, ldw,
                           k, (const uint32_t *)nullptr, (const int32_t *)nullptr,
                           (const int32_t *)nullptr, codes, scales, zeros, (int32_t *)nullptr,
                           (uint16_t *)nullptr, gs);
    }
    return hipGetLastError();
}

template <bool SYM>
static hipError_t quantize_mode(int bits, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                                int64_t kout, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                                int32_t *rowptr, int32_t *col, uint16_t *val, const QuantWs &ws,
                                hipStream_t st)
{
    switch (bits) {
    case 2: return quantize_bits<2, SYM>(w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    case 3: return quantize_bits<3, SYM>(w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    case 4: return quantize_bits<4, SYM>(w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    case 5: return quantize_bits<5, SYM>(w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    case 6: return quantize_bits<6, SYM>(w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(int bits, bool sym, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                           int64_t kout, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                           int32_t *rowptr, int32_t *col, uint16_t *val, const QuantWs &ws,
                           hipStream_t st)
{
    if (sym) return quantize_mode<true>(bits, w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
    return quantize_mode<false>(bits, w, ldw, n, k, gs, kout, codes, scales, zeros, rowptr, col, val, ws, st);
}

}  // namespace qp
