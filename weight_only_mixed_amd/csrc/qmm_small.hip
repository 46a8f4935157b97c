// Small-M dequant matmuls on gfx950 matrix cores: the decode GEMV (m <= 16) and the grouped
// routed-expert GEMM.
//
// The fused dequant-GEMM of the single-GPU 70B page (s3) is re-designed for CDNA4: packed
// weights stream from HBM with 16-byte loads straight into registers in the device tile
// order, every lane unpacks its own eight 8-k blocks (the page units, mixed-bit page s3.2)
// into exact fp16 (q - zp) values, and one v_mfma_f32_16x16x32_f16 per block multiplies 16
// weight rows by up to 16 activation rows.  Activation rows beyond m are zero, so the matrix
// core reduces over k for every m <= 16 at the same cost; no cross-lane shuffle reduction is
// needed inside a wave.  Each 128-k group is accumulated separately in fp32 and scaled by its
// fp16 scale in fp32 (mixed-bit page, s4.2).  The outlier CSR is added in fp32 before the one
// fp16 rounding of y (70B page, s2).
//
// Matrix-core fragment layout (A = 16 weight rows x 32 k, B = 32 k x 16 activation rows):
// lane l = 16*t + r supplies row r of A and column r of B for k-slots 8t..8t+7 and receives
// D[4t + i][r], i = 0..3 (weight row 4t+i, activation row r).
#include "unpack.h"

namespace qp {

__device__ __forceinline__ float lo_half(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
__device__ __forceinline__ float hi_half(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// All inputs of one k-tile for one lane: packed chunk, zero points of its A row, scales of
// its four output rows.
template <int B>
struct TileIn {
    uint32_t d[2 * B];
    uint32_t zz;     // two u8 zero points (groups 2kt, 2kt+1) of row 16*rb + r
    uint32_t sc[4];  // fp16 scales (2kt, 2kt+1) of rows 16*rb + 4t + i
};

template <int B>
__device__ __forceinline__ void load_tile(const ExpertPtrs &W, int64_t rb, int64_t kt, int64_t KT,
                                          int64_t G, int lane, TileIn<B> &in)
{
    const int t = lane >> 4, r = lane & 15;
    load_chunk<B>(W.packed + (rb * KT + kt) * (512 * B), lane, in.d);
    in.zz = *(const uint16_t *)(W.zeros + (rb * kTileN + r) * G + 2 * kt);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        in.sc[i] = *(const uint32_t *)(W.scales + (rb * kTileN + 4 * t + i) * G + 2 * kt);
}

__device__ __forceinline__ void load_x(const uint16_t *xrow, bool act, int64_t kt, int t, h8 *X)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (act)
            X[j] = *(const h8 *)(xrow + block_k0((int)kt, j, t));
        else
            X[j] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
    }
}

// tot += s0 * (A[0..3] . X[0..3]) + s1 * (A[4..7] . X[4..7]), groups kept apart.
__device__ __forceinline__ void mma_tile(const h8 *A, const h8 *X, const uint32_t *sc, f4 &tot)
{
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 a0 = mfma16(A[0], X[0], z);
    f4 a1 = mfma16(A[4], X[4], z);
    a0 = mfma16(A[1], X[1], a0);
    a1 = mfma16(A[5], X[5], a1);
    a0 = mfma16(A[2], X[2], a0);
    a1 = mfma16(A[6], X[6], a1);
    a0 = mfma16(A[3], X[3], a0);
    a1 = mfma16(A[7], X[7], a1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tot[i] = __builtin_fmaf(lo_half(sc[i]), a0[i], tot[i]);
        tot[i] = __builtin_fmaf(hi_half(sc[i]), a1[i], tot[i]);
    }
}

// ---- decode GEMV: one workgroup per 16-row block, NW waves split the k-tiles ----------
//
// Decode is latency-bound at these sizes (a 4096 x 4096 layer is a few MB), so each wave
// issues every global load it needs -- TPW weight tiles, their scales and zero points and
// the activation fragments -- before its first unpack, and the next chunk of TPW tiles is in
// flight while the current one is multiplied.  The NW partial sums of a row block are
// reduced through LDS in a fixed order.

template <int B, int TPW>
struct Chunk {
    TileIn<B> tile[TPW];
};

template <int B, int TPW>
__device__ __forceinline__ void load_w_chunk(const ExpertPtrs &W, int64_t rb, int64_t kt0, int64_t KT,
                                             int64_t G, int lane, Chunk<B, TPW> &c)
{
#pragma unroll
    for (int u = 0; u < TPW; ++u)
        if (kt0 + u < KT) load_tile<B>(W, rb, kt0 + u, KT, G, lane, c.tile[u]);
}

template <int TPW>
__device__ __forceinline__ void load_x_chunk(const uint16_t *xrow, bool act, int64_t kt0, int64_t KT, int t,
                                             h8 (&X)[TPW][8])
{
#pragma unroll
    for (int u = 0; u < TPW; ++u)
        if (kt0 + u < KT) load_x(xrow, act, kt0 + u, t, X[u]);
}

template <int B, int TPW>
__device__ __forceinline__ void compute_chunk(const Chunk<B, TPW> &c, const h8 (&X)[TPW][8], int64_t kt0,
                                              int64_t KT, f4 &tot)
{
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        if (kt0 + u < KT) {
            GroupConst<B> g0, g1;
            g0.set(c.tile[u].zz & 0xFF);
            g1.set((c.tile[u].zz >> 8) & 0xFF);
            h8 A[8];
            unpack_chunk<B>(c.tile[u].d, g0, g1, A);
            mma_tile(A, X[u], c.tile[u].sc, tot);
        }
    }
}

template <int B, int NW, int TPW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(SmallArgs a)
{
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t rb = blockIdx.x;
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;
    const ExpertPtrs &W = a.ex[0];
    const bool act = r < a.m;
    const uint16_t *xrow = a.x + (act ? r : 0) * a.ldx;
    constexpr int STRIDE = NW * TPW;

    f4 tot = {0.f, 0.f, 0.f, 0.f};
    Chunk<B, TPW> ca, cb;  // weight tiles: two named buffers, used alternately
    h8 X[TPW][8];          // activation fragments of the chunk being multiplied
    int64_t k0 = (int64_t)wv * TPW;
    if (k0 < KT) load_w_chunk<B, TPW>(W, rb, k0, KT, G, lane, ca);
    while (k0 < KT) {
        load_x_chunk<TPW>(xrow, act, k0, KT, t, X);
        if (k0 + STRIDE < KT) load_w_chunk<B, TPW>(W, rb, k0 + STRIDE, KT, G, lane, cb);
        compute_chunk<B, TPW>(ca, X, k0, KT, tot);
        k0 += STRIDE;
        if (k0 >= KT) break;
        load_x_chunk<TPW>(xrow, act, k0, KT, t, X);
        if (k0 + STRIDE < KT) load_w_chunk<B, TPW>(W, rb, k0 + STRIDE, KT, G, lane, ca);
        compute_chunk<B, TPW>(cb, X, k0, KT, tot);
        k0 += STRIDE;
    }

    __shared__ f4 red[NW][64];
    red[wv][lane] = tot;
    __syncthreads();
    if (wv != 0 || !act) return;
    f4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[w][lane];
    if (a.rowptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = rb * kTileN + 4 * t + i;
            for (int32_t p = a.rowptr[n]; p < a.rowptr[n + 1]; ++p) {
                const float xv = (float)__builtin_bit_cast(_Float16, xrow[a.col[p]]);
                const float wv16 = (float)__builtin_bit_cast(_Float16, a.val[p]);
                s[i] = __builtin_fmaf(xv, wv16, s[i]);
            }
        }
    }
    uint16_t *y = (uint16_t *)a.y + r * a.ldy + rb * kTileN + 4 * t;
    *(u2 *)y = (u2){pack_h2(s[0], s[1]), pack_h2(s[2], s[3])};
}

// ---- grouped experts: one wave per 16-row block (two for SwiGLU) over the whole k ------

template <int B, int EPI, int MT>
__global__ __launch_bounds__(256) void grouped_kernel(SmallArgs a)
{
    constexpr int RB = EPI == QP_EPI_SWIGLU ? 2 : 1;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int e = blockIdx.y;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wv;
    if (unit >= a.n / kTileN / RB) return;
    const int64_t r0 = a.offsets[e], r1 = a.offsets[e + 1];
    if (r1 <= r0) return;
    const ExpertPtrs &W = a.ex[e];
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;

    for (int64_t mb = r0; mb < r1; mb += 16 * MT) {
        const int nmt = (int)min<int64_t>(MT, (r1 - mb + 15) / 16);
        const uint16_t *xrow[MT];
        bool act[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t row = mb + 16 * mt + r;
            act[mt] = mt < nmt && row < r1;
            const int64_t tok = act[mt] ? (a.row_src ? a.row_src[row] : row) : 0;
            xrow[mt] = a.x + tok * a.ldx;
        }
        f4 tot[RB][MT];
#pragma unroll
        for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) tot[u][mt] = (f4){0.f, 0.f, 0.f, 0.f};

        TileIn<B> ta[RB], tb[RB];
        auto compute = [&](const TileIn<B> *in, int64_t kt) {
            h8 A[RB][8];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                GroupConst<B> g0, g1;
                g0.set(in[u].zz & 0xFF);
                g1.set((in[u].zz >> 8) & 0xFF);
                unpack_chunk<B>(in[u].d, g0, g1, A[u]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < nmt) {
                    h8 X[8];
                    load_x(xrow[mt], act[mt], kt, t, X);
#pragma unroll
                    for (int u = 0; u < RB; ++u) mma_tile(A[u], X, in[u].sc, tot[u][mt]);
                }
            }
        };
#pragma unroll
        for (int u = 0; u < RB; ++u) load_tile<B>(W, unit * RB + u, 0, KT, G, lane, ta[u]);
        for (int64_t kt = 0; kt < KT;) {
            if (kt + 1 < KT) {
#pragma unroll
                for (int u = 0; u < RB; ++u) load_tile<B>(W, unit * RB + u, kt + 1, KT, G, lane, tb[u]);
            }
            compute(ta, kt);
            if (++kt >= KT) break;
            if (kt + 1 < KT) {
#pragma unroll
                for (int u = 0; u < RB; ++u) load_tile<B>(W, unit * RB + u, kt + 1, KT, G, lane, ta[u]);
            }
            compute(tb, kt);
            ++kt;
        }

#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (!act[mt]) continue;
            const int64_t row = mb + 16 * mt + r;
            if constexpr (EPI == QP_EPI_NONE) {
                uint16_t *y = (uint16_t *)a.y + row * a.ldy + unit * kTileN + 4 * t;
                const f4 s = tot[0][mt];
                *(u2 *)y = (u2){pack_h2(s[0], s[1]), pack_h2(s[2], s[3])};
            } else if constexpr (EPI == QP_EPI_ROWS_F32) {
                float *y = (float *)a.y + row * a.ldy + unit * kTileN + 4 * t;
                *(f4 *)y = tot[0][mt];
            } else {
                const f4 g = tot[0][mt], u = tot[RB - 1][mt];
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
                uint16_t *y = (uint16_t *)a.y + row * a.ldy + unit * kTileN + 4 * t;
                *(u2 *)y = (u2){pack_h2(o[0], o[1]), pack_h2(o[2], o[3])};
            }
        }
    }
}

template <int B>
static hipError_t gemv_bits(const SmallArgs &a, hipStream_t st)
{
    constexpr int NW = 8, TPW = 1;
    hipLaunchKernelGGL((gemv_kernel<B, NW, TPW>), dim3((unsigned)(a.n / kTileN)), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemv(int bits, const SmallArgs &a, hipStream_t st)
{
    switch (bits) {
    case 2: return gemv_bits<2>(a, st);
    case 3: return gemv_bits<3>(a, st);
    case 4: return gemv_bits<4>(a, st);
    case 5: return gemv_bits<5>(a, st);
    case 6: return gemv_bits<6>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int B, int EPI>
static hipError_t grouped_epi(int n_experts, const SmallArgs &a, hipStream_t st)
{
    constexpr int RB = EPI == QP_EPI_SWIGLU ? 2 : 1;
    const int64_t units = a.n / kTileN / RB;
    const dim3 grid((unsigned)((units + 3) / 4), (unsigned)n_experts);
    hipLaunchKernelGGL((grouped_kernel<B, EPI, 8>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int B>
static hipError_t grouped_bits(int epi, int n_experts, const SmallArgs &a, hipStream_t st)
{
    switch (epi) {
    case QP_EPI_NONE: return grouped_epi<B, QP_EPI_NONE>(n_experts, a, st);
    case QP_EPI_SWIGLU: return grouped_epi<B, QP_EPI_SWIGLU>(n_experts, a, st);
    case QP_EPI_ROWS_F32: return grouped_epi<B, QP_EPI_ROWS_F32>(n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(int bits, int epi, int n_experts, const SmallArgs &a, hipStream_t st)
{
    switch (bits) {
    case 2: return grouped_bits<2>(epi, n_experts, a, st);
    case 3: return grouped_bits<3>(epi, n_experts, a, st);
    case 4: return grouped_bits<4>(epi, n_experts, a, st);
    case 5: return grouped_bits<5>(epi, n_experts, a, st);
    case 6: return grouped_bits<6>(epi, n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qp
