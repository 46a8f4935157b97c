// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  On CDNA4 the roles are split
// differently.  Each wave owns RBW 16-row weight blocks: it loads their packed tiles with
// 16-byte loads straight into registers (double-buffered across k-tiles) and unpacks them into
// exact fp16 (q - zp) A operands itself, so weights never pass through LDS and each weight is
// unpacked once per 128-row activation block.  The activation tile (128 rows x one 128-k
// group, 32 KB) is shared by the four waves through LDS: it is loaded with buffer-to-LDS DMA
// (no registers), double-buffered, with the 16-byte chunks of each row XOR-swizzled by the row
// index so the matrix-core fragment reads (16 rows, same column) hit distinct banks.  Every
// 128-k group is accumulated on the matrix cores in fp32 and then scaled by its fp16 scale in
// fp32.
//
// Outlier add-back (70B page, s2): the held-out fp16 weights are added in fp32 before the one
// fp16 rounding of y.  Two small kernels run first: one writes x transposed (x^T) into the
// caller's workspace, the other multiplies each weight row's outliers by it into an fp32
// sparse partial S^T[n][m].  The GEMM then starts its fp32 accumulators from S^T instead of
// zero, so the main loop is the same as without outliers.  Inside each 128-row block of m the
// transposed layouts keep row 16*mt + r at position 8*r + mt: a lane's eight accumulator rows
// (tiles mt = 0..7 of its row r) are 32 contiguous bytes of S^T.
//
// Workgroups are ordered so that the activation blocks of one weight tile run on the same XCD
// (block b runs on XCD b % 8), where they share that XCD's L2 copy of the packed weights.
#include "bufio.h"
#include "unpack.h"

namespace qp {

namespace {

constexpr int kWaves = 4;
constexpr int kRBW = 2;                      // 16-row weight blocks per wave
constexpr int kMT = 8;                       // 16-row activation tiles per workgroup
constexpr int kNT = kWaves * kRBW * kTileN;  // 128 weight rows per workgroup
constexpr int kMRows = kMT * 16;             // 128 activation rows per workgroup
constexpr int kRowBytes = 128 * 2;           // one 128-k group of one activation row

// LDS byte offset of 16-byte chunk c (8 k values) of activation row `row`.
__device__ __forceinline__ int xs_off(int row, int c) { return row * kRowBytes + ((c ^ (row & 15)) << 4); }

// Shared memory of one workgroup: the activation tiles (double buffer).
struct Smem {
    uint8_t xs[2][kMRows * kRowBytes];
};

// Buffers of one workgroup.  Every wave-uniform offset passed as soffset stays inside the
// range the per-lane voffset was checked against (a row of x, a weight row block), so a
// load is in bounds whether or not the hardware includes soffset in its range check.
struct Bufs {
    rsrc_t x;              // activation rows [m0, m)
    rsrc_t w[kRBW];        // packed tiles of row block rb0 + u (empty past the last block)
    rsrc_t sc[kRBW], zr[kRBW];
    uint32_t xoff[8];      // this lane's source of LDS-DMA piece it (row offset + chunk)
};

// DMA the 128 x 128-k activation tile of group g into LDS buffer `dst` (this wave's 8 KB).
// Lane L of piece `it` fills LDS bytes [16L, 16L+16) of a 1 KB run = row 4*(8*wv+it) + L/16,
// physical chunk L%16, which holds logical chunk (L%16) ^ (row & 15).
__device__ __forceinline__ void dma_x(const Bufs &bf, int64_t g, uint8_t *dst, int wv)
{
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)g * 256);  // column of group g
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        uint8_t *base = dst + (wv * 8 + it) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bf.x, (__attribute__((address_space(3))) void *)base, 16,
                                                 bf.xoff[it], soff, 0, 0);
    }
}

__device__ __forceinline__ void wait_dma_and_sync()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

template <int B>
struct WTile {
    uint32_t d[kRBW][2 * B];
    uint32_t zz[kRBW];
    uint32_t sc[kRBW][4];
};

// Weight tile kt of this wave's row blocks.
template <int B>
__device__ __forceinline__ void load_w(const Bufs &bf, int64_t G, int64_t kt, int lane, WTile<B> &w)
{
    const int t = lane >> 4, r = lane & 15;
    const uint32_t vw = 16 * lane, vw8 = 8 * lane;
    const uint32_t vz = (uint32_t)(r * G), vs = (uint32_t)(4 * t * G * 2);
    const uint32_t tile = __builtin_amdgcn_readfirstlane((uint32_t)(kt * (512 * B)));
    const uint32_t zo = __builtin_amdgcn_readfirstlane((uint32_t)(2 * kt));
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
#pragma unroll
        for (int sl = 0; sl < B / 2; ++sl) {
            const u4 v = ld16(bf.w[u], vw, tile + 1024 * sl);
            w.d[u][4 * sl + 0] = v[0];
            w.d[u][4 * sl + 1] = v[1];
            w.d[u][4 * sl + 2] = v[2];
            w.d[u][4 * sl + 3] = v[3];
        }
        if (B & 1) {
            const u2 v = ld8(bf.w[u], vw8, tile + 1024 * (B / 2));
            w.d[u][2 * B - 2] = v[0];
            w.d[u][2 * B - 1] = v[1];
        }
        w.zz[u] = ld2(bf.zr[u], vz, zo);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w.sc[u][i] = ld4(bf.sc[u], vs, __builtin_amdgcn_readfirstlane((uint32_t)((i * G + 2 * kt) * 2)));
    }
}

// One 128-k group: unpack this wave's four blocks of group gi for each row block, multiply by
// the eight activation tiles from LDS, scale and accumulate.
template <int B, int GI>
__device__ __forceinline__ void group_step(const WTile<B> &w, const uint8_t *xs, int lane,
                                           f4 (&tot)[kRBW][kMT])
{
    const int t = lane >> 4, r = lane & 15;
    h8 A[kRBW][4];
    float s[kRBW][4];
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        GroupConst<B> gc;
        gc.set(GI == 0 ? (w.zz[u] & 0xFF) : ((w.zz[u] >> 8) & 0xFF));
        A[u][0] = BlockUnpack<B, 4 * GI + 0>::run(w.d[u], gc);
        A[u][1] = BlockUnpack<B, 4 * GI + 1>::run(w.d[u], gc);
        A[u][2] = BlockUnpack<B, 4 * GI + 2>::run(w.d[u], gc);
        A[u][3] = BlockUnpack<B, 4 * GI + 3>::run(w.d[u], gc);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[u][i] = GI == 0 ? lo_h(w.sc[u][i]) : hi_h(w.sc[u][i]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        const int row = 16 * mt + r;
        h8 X[4];
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) X[j4] = *(const h8 *)(xs + xs_off(row, 4 * j4 + t));
        f4 acc[kRBW];
#pragma unroll
        for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][0], X[0], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j4 = 1; j4 < 4; ++j4)
#pragma unroll
            for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][j4], X[j4], acc[u]);
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[u][mt][i] = __builtin_fmaf(s[u][i], acc[u][i], tot[u][mt][i]);
            // Pin the update here: without it the compiler sinks these fmas below later tiles,
            // keeping every tile's matrix-core result live at once.
            asm volatile("" : "+v"(tot[u][mt]));
        }
        // keep the next tile's fragment reads from being hoisted above this point (register
        // pressure); the other wave on the SIMD covers the LDS latency
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace

template <int B, bool OUTL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) Smem sm;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, m_tiles = (a.m + kMRows - 1) / kMRows;
    int64_t nt, mtile;
    const int64_t b = blockIdx.x;
    if (n_tiles % 8 == 0) {  // XCD-aware: the m blocks of one n tile share an XCD
        const int64_t xcd = b % 8, local = b / 8;
        nt = (local / m_tiles) * 8 + xcd;
        mtile = local % m_tiles;
    } else {
        nt = b % n_tiles;
        mtile = b / n_tiles;
    }
    const int64_t m0 = mtile * kMRows;
    const int64_t NB = a.n / kTileN;
    const int64_t n0 = nt * kNT;                          // first weight row of the workgroup
    const int64_t rb0 = nt * (kNT / kTileN) + wv * kRBW;  // first row block of this wave

    Bufs bf;
    bf.x = make_rsrc(a.x + m0 * a.ldx, (a.m - m0) * a.ldx * 2);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = 32 * wv + 4 * it + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        bf.xoff[it] = (uint32_t)((row * a.ldx + 8 * c) * 2);
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        const bool in = rb < NB;
        bf.w[u] = make_rsrc(a.packed + rb * KT * (512 * B), in ? KT * (512 * B) : 0);
        bf.sc[u] = make_rsrc(a.scales + rb * kTileN * G, in ? kTileN * G * 2 : 0);
        bf.zr[u] = make_rsrc(a.zeros + rb * kTileN * G, in ? kTileN * G : 0);
    }

    f4 tot[kRBW][kMT];
    if constexpr (OUTL) {
        // accumulators start from the outlier partial S^T (rows past n read as zeros)
        const rsrc_t sr = make_rsrc(a.spart, a.n * a.ldxt * 4);
        const uint32_t ld = (uint32_t)(a.ldxt * 4);
        const uint32_t v0 = (uint32_t)(((rb0 * kTileN + 4 * t) * a.ldxt + m0 + 8 * r) * 4);
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
            u4 lo[4], hi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = v0 + (uint32_t)(u * kTileN + i) * ld;
                lo[i] = ld16(sr, off);
                hi[i] = ld16(sr, off + 16);
            }
            // whole-vector construction (element-wise stores into an unset vector are avoided)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                tot[u][mt] = (f4){as_f(lo[0][mt]), as_f(lo[1][mt]), as_f(lo[2][mt]), as_f(lo[3][mt])};
                tot[u][mt + 4] = (f4){as_f(hi[0][mt]), as_f(hi[1][mt]), as_f(hi[2][mt]), as_f(hi[3][mt])};
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < kRBW; ++u)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                tot[u][mt] = (f4){0.f, 0.f, 0.f, 0.f};
                // opaque zero: a known-zero start lets the compiler specialise the first group
                // steps, which costs registers across the whole loop
                asm volatile("" : "+v"(tot[u][mt]));
            }
    }

    dma_x(bf, 0, sm.xs[0], wv);
    WTile<B> wa, wb;
    load_w<B>(bf, G, 0, lane, wa);
    wait_dma_and_sync();

    // Two k-tiles (four groups) per iteration so both weight buffers are named statically.
    for (int64_t kt = 0; kt < KT; kt += 2) {
        // group 2kt (LDS buffer 0): prefetch group 2kt+1 activations and the next weight tile
        dma_x(bf, 2 * kt + 1, sm.xs[1], wv);
        if (kt + 1 < KT) load_w<B>(bf, G, kt + 1, lane, wb);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0>(wa, sm.xs[0], lane, tot);
        wait_dma_and_sync();
        // group 2kt+1 (buffer 1)
        if (kt + 1 < KT) dma_x(bf, 2 * kt + 2, sm.xs[0], wv);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1>(wa, sm.xs[1], lane, tot);
        wait_dma_and_sync();
        if (kt + 1 >= KT) break;
        // group 2kt+2 (buffer 0)
        dma_x(bf, 2 * kt + 3, sm.xs[1], wv);
        if (kt + 2 < KT) load_w<B>(bf, G, kt + 2, lane, wa);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0>(wb, sm.xs[0], lane, tot);
        wait_dma_and_sync();
        // group 2kt+3 (buffer 1)
        if (kt + 2 < KT) dma_x(bf, 2 * kt + 4, sm.xs[0], wv);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1>(wb, sm.xs[1], lane, tot);
        wait_dma_and_sync();
    }

    // epilogue: the fp16 store
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        if (rb >= NB) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int64_t row = m0 + 16 * mt + r;
            if (row >= a.m) continue;
            const f4 s = tot[u][mt];
            uint16_t *y = a.y + row * a.ldy + rb * kTileN + 4 * t;
            *(u2 *)y = (u2){pack_h2(s[0], s[1]), pack_h2(s[2], s[3])};
        }
    }
}

// x^T for the outlier gathers: xt[kk][128 mb + 8 r + mt] = x[128 mb + 16 mt + r][kk], zeros for
// rows >= m.  One block per 64 k x 128 m tile, staged through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                                                        uint16_t *xt, int64_t ldxt)
{
    __shared__ uint16_t tile[128][65];
    const int64_t k0 = blockIdx.x * 64, m0 = blockIdx.y * 128;
    for (int i = threadIdx.x; i < 128 * 64; i += 256) {
        const int rm = i / 64, ck = i % 64;
        const int64_t gm = m0 + rm, gk = k0 + ck;
        tile[rm][ck] = (gm < m && gk < k) ? x[gm * ldx + gk] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 128 * 64; i += 256) {
        const int rk = i / 128, pos = i % 128;      // pos = 8 r + mt holds row 16 mt + r
        const int rm = 16 * (pos & 7) + (pos >> 3);
        const int64_t gk = k0 + rk;
        if (gk < k) xt[gk * ldxt + m0 + pos] = tile[rm][rk];
    }
}

// Outlier partial: S^T[n][p] = sum over the outliers (n, c, v) of v * x^T[c][p], in fp32 (one
// wave per weight row, each lane 8 consecutive positions p of a 512-position chunk).
__global__ __launch_bounds__(256) void outlier_spmm_kernel(const int32_t *rowptr, const int32_t *col,
                                                           const uint16_t *val, const uint16_t *xt, int64_t n,
                                                           int64_t ldxt, float *spart)
{
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wv;
    const int64_t p = (int64_t)blockIdx.y * 512 + 8 * lane;
    if (row >= n || p >= ldxt) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t e0 = rowptr[row], e1 = rowptr[row + 1];
    for (int64_t e = e0; e < e1; ++e) {
        const float v = h_f(val[e]);
        const u4 xv = *(const u4 *)(xt + (int64_t)col[e] * ldxt + p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] = __builtin_fmaf(lo_h(xv[j]), v, acc[2 * j]);
            acc[2 * j + 1] = __builtin_fmaf(hi_h(xv[j]), v, acc[2 * j + 1]);
        }
    }
    f4 *dst = (f4 *)(spart + row * ldxt + p);
    dst[0] = (f4){acc[0], acc[1], acc[2], acc[3]};
    dst[1] = (f4){acc[4], acc[5], acc[6], acc[7]};
}

template <int B>
static hipError_t gemm_bits(const GemmArgs &a, hipStream_t st)
{
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, m_tiles = (a.m + kMRows - 1) / kMRows;
    if (a.rowptr) {
        hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((a.k + 63) / 64), (unsigned)(a.ldxt / 128)), dim3(256), 0,
                           st, a.x, a.ldx, a.m, a.k, a.xt, a.ldxt);
        hipLaunchKernelGGL(outlier_spmm_kernel, dim3((unsigned)((a.n + 3) / 4), (unsigned)((a.ldxt + 511) / 512)),
                           dim3(256), 0, st, a.rowptr, a.col, a.val, a.xt, a.n, a.ldxt, a.spart);
        hipLaunchKernelGGL((gemm_kernel<B, true>), dim3((unsigned)(n_tiles * m_tiles)), dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL((gemm_kernel<B, false>), dim3((unsigned)(n_tiles * m_tiles)), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

int64_t gemm_xt_ld(int64_t m) { return (m + kMRows - 1) / kMRows * kMRows; }

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
