// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  On CDNA4 the roles are split
// differently.  Each wave owns RBW 16-row weight blocks: it loads their packed tiles with
// 16-byte loads straight into registers (double-buffered across k-tiles) and unpacks them into
// exact fp16 (q - zp) A operands itself, so weights never pass through LDS and each weight is
// unpacked once per 128-row activation block.  The activation tile (128 rows x one 128-k
// group, 32 KB) is shared by the four waves through LDS, double-buffered, with the 16-byte
// chunks of each row XOR-swizzled by the row index so that the matrix-core fragment reads
// (16 rows, same column) hit distinct banks.  Every 128-k group is accumulated on the matrix
// cores in fp32 and then scaled by its fp16 scale in fp32; the outlier CSR is added in the
// epilogue before the single fp16 rounding of y.
//
// Workgroups are ordered so that the activation blocks of one weight tile run on the same XCD
// (block b runs on XCD b % 8), where they share that XCD's L2 copy of the packed weights.
#include "unpack.h"

namespace qp {

namespace {

constexpr int kWaves = 4;
constexpr int kRBW = 2;                      // 16-row weight blocks per wave
constexpr int kMT = 8;                       // 16-row activation tiles per workgroup
constexpr int kNT = kWaves * kRBW * kTileN;  // 128 weight rows per workgroup
constexpr int kMRows = kMT * 16;             // 128 activation rows per workgroup
constexpr int kRowBytes = 128 * 2;           // one 128-k group of one activation row

__device__ __forceinline__ float lo_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
__device__ __forceinline__ float hi_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// LDS byte offset of 16-byte chunk c (8 k values) of activation row `row`.
__device__ __forceinline__ int xs_off(int row, int c) { return row * kRowBytes + ((c ^ (row & 15)) << 4); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zeros.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ u4 ld16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u2 ld8(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ uint32_t ld2(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0); }

// Buffers of one workgroup: activation rows m0.. (rows past m read as zeros) and the weight
// rows of this wave's blocks.
struct Bufs {
    rsrc_t x, w, sc, zr;
    uint32_t xoff;    // this thread's first activation piece (row tid/16, chunk tid%16)
    uint32_t xrow16;  // bytes between activation rows 16 apart
};

// This thread's 8 pieces of the 128 x 128-k activation tile of group `g`.
__device__ __forceinline__ void load_x(const Bufs &bf, int64_t g, u4 *buf)
{
#pragma unroll
    for (int it = 0; it < 8; ++it) buf[it] = ld16(bf.x, bf.xoff + it * bf.xrow16 + (uint32_t)g * 256);
}

__device__ __forceinline__ void store_x(uint8_t *lds, const u4 *buf)
{
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        *(u4 *)(lds + xs_off(idx >> 4, idx & 15)) = buf[it];
    }
}

template <int B>
struct WTile {
    uint32_t d[kRBW][2 * B];
    uint32_t zz[kRBW];
    uint32_t sc[kRBW][4];
};

// Weight tile kt of this wave's row blocks (offsets relative to the wave's first block).
template <int B>
__device__ __forceinline__ void load_w(const Bufs &bf, int64_t KT, int64_t G, int64_t kt, int lane, WTile<B> &w)
{
    const int t = lane >> 4, r = lane & 15;
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const uint32_t tile = (uint32_t)((u * KT + kt) * (512 * B));
#pragma unroll
        for (int sl = 0; sl < B / 2; ++sl) {
            const u4 v = ld16(bf.w, tile + 1024 * sl + 16 * lane);
            w.d[u][4 * sl + 0] = v[0];
            w.d[u][4 * sl + 1] = v[1];
            w.d[u][4 * sl + 2] = v[2];
            w.d[u][4 * sl + 3] = v[3];
        }
        if (B & 1) {
            const u2 v = ld8(bf.w, tile + 1024 * (B / 2) + 8 * lane);
            w.d[u][2 * B - 2] = v[0];
            w.d[u][2 * B - 1] = v[1];
        }
        w.zz[u] = ld2(bf.zr, (uint32_t)((u * kTileN + r) * G + 2 * kt));
#pragma unroll
        for (int i = 0; i < 4; ++i) w.sc[u][i] = ld4(bf.sc, (uint32_t)(((u * kTileN + 4 * t + i) * G + 2 * kt) * 2));
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

template <int B>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][kMRows * kRowBytes];
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
    const int64_t rb0 = nt * (kNT / kTileN) + wv * kRBW;
    const int64_t nrb = NB - rb0;  // row blocks from this wave's first to the end of W

    Bufs bf;
    bf.x = make_rsrc(a.x + m0 * a.ldx, (a.m - m0) * a.ldx * 2);
    bf.xoff = (uint32_t)(((threadIdx.x >> 4) * a.ldx + 8 * (threadIdx.x & 15)) * 2);
    bf.xrow16 = (uint32_t)(16 * a.ldx * 2);
    bf.w = make_rsrc(a.packed + rb0 * KT * (512 * B), nrb * KT * (512 * B));
    bf.sc = make_rsrc(a.scales + rb0 * kTileN * G, nrb * kTileN * G * 2);
    bf.zr = make_rsrc(a.zeros + rb0 * kTileN * G, nrb * kTileN * G);

    f4 tot[kRBW][kMT];
#pragma unroll
    for (int u = 0; u < kRBW; ++u)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) tot[u][mt] = (f4){0.f, 0.f, 0.f, 0.f};

    u4 xbuf[8];
    load_x(bf, 0, xbuf);
    store_x(xs[0], xbuf);
    WTile<B> wa, wb;
    load_w<B>(bf, KT, G, 0, lane, wa);
    __syncthreads();

    // Two k-tiles (four groups) per iteration so both weight buffers are named statically.
    // Scheduling barriers keep each group step's unpack and fragment reads inside its step.
    for (int64_t kt = 0; kt < KT; kt += 2) {
        // group 2kt (buffer 0): prefetch group 2kt+1 activations and the next weight tile
        load_x(bf, 2 * kt + 1, xbuf);
        if (kt + 1 < KT) load_w<B>(bf, KT, G, kt + 1, lane, wb);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0>(wa, xs[0], lane, tot);
        store_x(xs[1], xbuf);
        __syncthreads();
        // group 2kt+1 (buffer 1)
        if (kt + 1 < KT) load_x(bf, 2 * kt + 2, xbuf);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1>(wa, xs[1], lane, tot);
        if (kt + 1 < KT) store_x(xs[0], xbuf);
        __syncthreads();
        if (kt + 1 >= KT) break;
        // group 2kt+2 (buffer 0)
        load_x(bf, 2 * kt + 3, xbuf);
        if (kt + 2 < KT) load_w<B>(bf, KT, G, kt + 2, lane, wa);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0>(wb, xs[0], lane, tot);
        store_x(xs[1], xbuf);
        __syncthreads();
        // group 2kt+3 (buffer 1)
        if (kt + 2 < KT) load_x(bf, 2 * kt + 4, xbuf);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1>(wb, xs[1], lane, tot);
        if (kt + 2 < KT) store_x(xs[0], xbuf);
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
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, m_tiles = (a.m + kMRows - 1) / kMRows;
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
