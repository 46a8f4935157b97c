// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  Here the roles are re-assigned for
// CDNA4: each wave owns RBW 16-row weight blocks and unpacks them straight from its own
// 16-byte loads of the device tile order into fp16 A operands (no LDS round trip for the
// weights, each weight is unpacked once per 128-row activation block), while the
// activation tile, shared by all waves of the workgroup, is staged through LDS one 128-k
// group at a time (double-buffered).  Each 128-k group is accumulated in fp32 on the matrix
// cores and then scaled by its fp16 scale in fp32; the outlier CSR is added in the epilogue
// before the single fp16 rounding.
#include "unpack.h"

namespace qp {

namespace {

constexpr int kWaves = 4;
constexpr int kRBW = 4;          // 16-row weight blocks per wave
constexpr int kMT = 8;           // 16-row activation tiles per workgroup (128 rows)
constexpr int kNT = kWaves * kRBW * kTileN;  // 256 weight rows per workgroup
constexpr int kPitch = 128 * 2 + 16;         // LDS row pitch (bytes) of one 128-k group

__device__ __forceinline__ float lo_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
__device__ __forceinline__ float hi_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Global -> registers: this thread's 8 x 16-byte pieces of a 128-row x 128-k activation tile.
__device__ __forceinline__ void load_xstage(const uint16_t *x, int64_t ldx, int64_t m,
                                            int64_t m0, int64_t k0, u4 *buf)
{
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, ch = idx & 15;
        const int64_t gm = m0 + row;
        if (gm < m)
            buf[it] = *(const u4 *)(x + gm * ldx + k0 + 8 * ch);
        else
            buf[it] = (u4){0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_xstage(uint8_t *lds, const u4 *buf)
{
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, ch = idx & 15;
        *(u4 *)(lds + row * kPitch + 16 * ch) = buf[it];
    }
}

}  // namespace

template <int B>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][128 * kPitch];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;
    const int64_t n_tiles = (a.n + kNT - 1) / kNT;
    const int64_t nt = blockIdx.x % n_tiles, mtile = blockIdx.x / n_tiles;
    const int64_t m0 = mtile * 128;
    const int64_t rb0 = nt * (kNT / kTileN) + wv * kRBW;  // first row block of this wave
    const int64_t NB = a.n / kTileN;

    f4 tot[kRBW][kMT];
#pragma unroll
    for (int u = 0; u < kRBW; ++u)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) tot[u][mt] = (f4){0.f, 0.f, 0.f, 0.f};

    uint32_t d[kRBW][2 * B];
    uint32_t zz[kRBW];
    uint32_t sc[kRBW][4];
    auto load_w = [&](int64_t kt) {
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
            const int64_t rb = rb0 + u;
            if (rb < NB) {
                load_chunk<B>(a.packed + (rb * KT + kt) * (512 * B), lane, d[u]);
                zz[u] = *(const uint16_t *)(a.zeros + (rb * kTileN + r) * G + 2 * kt);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[u][i] = *(const uint32_t *)(a.scales + (rb * kTileN + 4 * t + i) * G + 2 * kt);
            } else {
#pragma unroll
                for (int q = 0; q < 2 * B; ++q) d[u][q] = 0;
                zz[u] = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[u][i] = 0;
            }
        }
    };

    u4 xbuf[8];
    load_xstage(a.x, a.ldx, a.m, m0, 0, xbuf);
    store_xstage(xs[0], xbuf);
    __syncthreads();
    load_w(0);

    const int64_t stages = 2 * KT;  // one stage = one 128-k group
    for (int64_t sidx = 0; sidx < stages; ++sidx) {
        const int gi = (int)(sidx & 1);
        const int64_t kt = sidx >> 1;
        const uint8_t *xcur = xs[sidx & 1];
        if (sidx + 1 < stages) load_xstage(a.x, a.ldx, a.m, m0, (sidx + 1) * 128, xbuf);

        // unpack this group's four blocks for every row block of the wave
        h8 A[kRBW][4];
        float s_lo[kRBW][4];
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
            GroupConst<B> gc;
            gc.set(gi == 0 ? (zz[u] & 0xFF) : ((zz[u] >> 8) & 0xFF));
            if (gi == 0) {
                A[u][0] = BlockUnpack<B, 0>::run(d[u], gc);
                A[u][1] = BlockUnpack<B, 1>::run(d[u], gc);
                A[u][2] = BlockUnpack<B, 2>::run(d[u], gc);
                A[u][3] = BlockUnpack<B, 3>::run(d[u], gc);
            } else {
                A[u][0] = BlockUnpack<B, 4>::run(d[u], gc);
                A[u][1] = BlockUnpack<B, 5>::run(d[u], gc);
                A[u][2] = BlockUnpack<B, 6>::run(d[u], gc);
                A[u][3] = BlockUnpack<B, 7>::run(d[u], gc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) s_lo[u][i] = gi == 0 ? lo_h(sc[u][i]) : hi_h(sc[u][i]);
        }
        if (gi == 1 && kt + 1 < KT) load_w(kt + 1);

#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            h8 X[4];
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4)
                X[j4] = *(const h8 *)(xcur + (16 * mt + r) * kPitch + 64 * j4 + 16 * t);
            f4 acc[kRBW];
#pragma unroll
            for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][0], X[0], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j4 = 1; j4 < 4; ++j4)
#pragma unroll
                for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][j4], X[j4], acc[u]);
#pragma unroll
            for (int u = 0; u < kRBW; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[u][mt][i] = __builtin_fmaf(s_lo[u][i], acc[u][i], tot[u][mt][i]);
        }

        if (sidx + 1 < stages) {
            store_xstage(xs[(sidx + 1) & 1], xbuf);
        }
        __syncthreads();
    }

    // epilogue: outlier add-back, fp16 store
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        if (rb >= NB) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int64_t row = m0 + 16 * mt + r;
            if (row >= a.m) continue;
            f4 s = tot[u][mt];
            if (a.rowptr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t n = rb * kTileN + 4 * t + i;
                    for (int32_t p = a.rowptr[n]; p < a.rowptr[n + 1]; ++p) {
                        const float xv = (float)__builtin_bit_cast(_Float16, a.x[row * a.ldx + a.col[p]]);
                        s[i] = __builtin_fmaf(xv, (float)__builtin_bit_cast(_Float16, a.val[p]), s[i]);
                    }
                }
            }
            uint16_t *y = a.y + row * a.ldy + rb * kTileN + 4 * t;
            *(u2 *)y = (u2){pack2(s[0], s[1]), pack2(s[2], s[3])};
        }
    }
}

template <int B>
static hipError_t gemm_bits(const GemmArgs &a, hipStream_t st)
{
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, m_tiles = (a.m + 127) / 128;
    hipLaunchKernelGGL((gemm_kernel<B>), dim3((unsigned)(n_tiles * m_tiles)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm(int bits, const GemmArgs &a, hipStream_t st)
{
    switch (bits) {
    case 2: return gemm_bits<2>(a, st);
    case 3: return gemm_bits<3>(a, st);
    case 4: return gemm_bits<4>(a, st);
    case 5: return gemm_bits<5>(a, st);
    case 6: return gemm_bits<6>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qp
