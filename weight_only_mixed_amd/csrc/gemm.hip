// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  On CDNA4 the roles are split
// differently.  Each of the eight waves of a workgroup owns two 16-row weight blocks: it loads
// their packed tiles with 16-byte loads straight into registers (one k-tile ahead) and unpacks
// them into exact fp16 (q - zp) A operands itself, so weights never pass through LDS and each
// weight is unpacked once per 128-row activation block.  The activation tile (128 rows x one
// 128-k group, 32 KB) is shared by the eight waves (256 weight rows) through a four-slot LDS
// ring filled by buffer-to-LDS DMA three groups ahead (no registers), with the 16-byte chunks
// of each row XOR-swizzled by the row index so the matrix-core fragment reads (16 rows, same
// column) hit distinct banks.  Every 128-k group is accumulated on the matrix cores in fp32
// and then scaled by its fp16 scale in fp32.
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

constexpr int kWaves = 8;
constexpr int kRBW = 2;                      // 16-row weight blocks per wave
constexpr int kMT = 8;                       // 16-row activation tiles per workgroup
constexpr int kNT = kWaves * kRBW * kTileN;  // 256 weight rows per workgroup
constexpr int kRing = 4;                     // activation ring slots
constexpr int kAhead = kRing - 1;            // groups the activation DMA runs ahead
constexpr int kDmaOps = 4;                   // DMA instructions per wave per group
constexpr int kMRows = kMT * 16;             // 128 activation rows per workgroup
constexpr int kRowBytes = 128 * 2;           // one 128-k group of one activation row

// LDS byte offset of 16-byte chunk c (8 k values) of activation row `row`.
__device__ __forceinline__ int xs_off(int row, int c) { return row * kRowBytes + ((c ^ (row & 15)) << 4); }

// Shared memory of one workgroup: the activation ring.
struct Smem {
    uint8_t xs[kRing][kMRows * kRowBytes];
};

// Buffers of one workgroup.  Every wave-uniform offset passed as soffset stays inside the
// range the per-lane voffset was checked against (a row of x, a weight row block), so a
// load is in bounds whether or not the hardware includes soffset in its range check.
struct Bufs {
    rsrc_t x;              // activation rows [m0, m)
    rsrc_t w[kRBW];        // packed tiles of row block rb0 + u (empty past the last block)
    rsrc_t sc[kRBW], zr[kRBW];
    uint32_t xoff[kDmaOps];  // this lane's source of LDS-DMA piece it (row offset + chunk)
};

// DMA the 128 x 128-k activation tile of group g into LDS slot `dst` (this wave's 4 KB).
// Lane L of piece `it` fills LDS bytes [16L, 16L+16) of a 1 KB run = row 4*(4*wv+it) + L/16,
// physical chunk L%16, which holds logical chunk (L%16) ^ (row & 15).
__device__ __forceinline__ void dma_x(const Bufs &bf, int64_t g, uint8_t *dst, int wv)
{
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)g * 256);  // column of group g
#pragma unroll
    for (int it = 0; it < kDmaOps; ++it) {
        uint8_t *base = dst + (wv * kDmaOps + it) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bf.x, (__attribute__((address_space(3))) void *)base, 16,
                                                 bf.xoff[it], soff, 0, 0);
    }
}

// Loads issued by load_w<B> (per row block: the packed pieces, one zero-point load, four
// scale loads).
template <int B>
constexpr int kLoadWOps = kRBW * (B / 2 + (B & 1) + 5);

// Wait until at most N of this wave's loads are outstanding (they retire in order), then
// synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_and_sync()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// One 128-k group: unpack this wave's four blocks of group GI for each row block, then
// multiply them by the eight 16-row activation tiles from LDS, scale and accumulate.  The
// tile loop is software-pipelined: the fragment reads of tile mt+1 are issued before the
// matrix-core chain of tile mt, and the fp32 scale-accumulate of tile mt-1 runs on the
// vector ALU while that chain executes.
template <int B, int GI, bool FULL>
__device__ __forceinline__ void group_step(const WTile<B> &w, const uint8_t *xs, int lane, int nmt,
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
    h8 X[2][4];
    f4 acc[2][kRBW];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) X[0][j4] = *(const h8 *)(xs + xs_off(r, 4 * j4 + t));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (!FULL && mt >= nmt) break;  // uniform: tiles past the workgroup's rows are skipped
        const int cur = mt & 1, nxt = cur ^ 1;
        if (mt + 1 < kMT && (FULL || mt + 1 < nmt)) {
            const int row = 16 * (mt + 1) + r;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) X[nxt][j4] = *(const h8 *)(xs + xs_off(row, 4 * j4 + t));
        }
        // keep the reads ahead of the chain (else they reuse the chain's fragment registers
        // and issue too late to hide their latency)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kRBW; ++u) acc[cur][u] = mfma16(A[u][0], X[cur][0], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j4 = 1; j4 < 4; ++j4)
#pragma unroll
            for (int u = 0; u < kRBW; ++u) acc[cur][u] = mfma16(A[u][j4], X[cur][j4], acc[cur][u]);
        if (mt > 0) {
#pragma unroll
            for (int u = 0; u < kRBW; ++u) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tot[u][mt - 1][i] = __builtin_fmaf(s[u][i], acc[nxt][u][i], tot[u][mt - 1][i]);
                asm volatile("" : "+v"(tot[u][mt - 1]));
            }
        }
        if (FULL ? mt + 1 == kMT : mt + 1 == nmt) {  // the last tile's scale-accumulate
#pragma unroll
            for (int u = 0; u < kRBW; ++u) {
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[u][mt][i] = __builtin_fmaf(s[u][i], acc[cur][u][i], tot[u][mt][i]);
                asm volatile("" : "+v"(tot[u][mt]));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The k loop of a workgroup.  Activation ring: the tile of group g sits in slot g % kRing; the
// DMA of group g + kAhead is issued at the start of step g (groups past the end reload the
// last one into a slot that is never read, and weight tiles past the end reload the last
// tile into the idle register buffer), so every step issues the same loads and the wait
// counts are fixed.  Order of a wave's loads: [DMA g+3] then, on even g, [weights of tile
// g/2 + 1].  The tile of group g+1 is needed after step g; the loads younger than its DMA
// (issued at step g-2) are the DMAs of g+2 and g+3 plus the weight batches of the even
// steps among g-2, g-1, g.  FULL: all eight 16-row activation tiles hold rows.
template <int B, bool FULL>
__device__ __forceinline__ void k_loop(const Bufs &bf, Smem &sm, int64_t KT, int64_t G, int wv, int lane, int nmt,
                                       f4 (&tot)[kRBW][kMT])
{
    const int64_t GN = 2 * KT;  // groups
    auto gclamp = [&](int64_t g) { return g < GN ? g : GN - 1; };
    auto tclamp = [&](int64_t t) { return t < KT ? t : KT - 1; };
    WTile<B> wa, wb;
    dma_x(bf, 0, sm.xs[0], wv);
    dma_x(bf, gclamp(1), sm.xs[1], wv);
    __builtin_amdgcn_sched_barrier(0);
    load_w<B>(bf, G, 0, lane, wa);
    __builtin_amdgcn_sched_barrier(0);
    dma_x(bf, gclamp(2), sm.xs[2], wv);
    wait_and_sync<kDmaOps>();  // group 0's DMA and tile 0's weights are in

    // Two k-tiles (four groups) per iteration so both weight buffers are named statically.
    for (int64_t kt = 0; kt < KT; kt += 2) {
        const int64_t g = 2 * kt;
        // group g (tile kt, first half): fetch tile kt+1's weights
        dma_x(bf, gclamp(g + 3), sm.xs[(g + 3) % kRing], wv);
        __builtin_amdgcn_sched_barrier(0);
        load_w<B>(bf, G, tclamp(kt + 1), lane, wb);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0, FULL>(wa, sm.xs[g % kRing], lane, nmt, tot);
        wait_and_sync<2 * kDmaOps + 2 * kLoadWOps<B>>();
        // group g+1 (tile kt, second half)
        dma_x(bf, gclamp(g + 4), sm.xs[(g + 4) % kRing], wv);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1, FULL>(wa, sm.xs[(g + 1) % kRing], lane, nmt, tot);
        wait_and_sync<2 * kDmaOps + kLoadWOps<B>>();
        if (kt + 1 >= KT) break;
        // group g+2 (tile kt+1, first half): fetch tile kt+2's weights
        dma_x(bf, gclamp(g + 5), sm.xs[(g + 5) % kRing], wv);
        __builtin_amdgcn_sched_barrier(0);
        load_w<B>(bf, G, tclamp(kt + 2), lane, wa);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 0, FULL>(wb, sm.xs[(g + 2) % kRing], lane, nmt, tot);
        wait_and_sync<2 * kDmaOps + 2 * kLoadWOps<B>>();
        // group g+3 (tile kt+1, second half)
        dma_x(bf, gclamp(g + 6), sm.xs[(g + 6) % kRing], wv);
        __builtin_amdgcn_sched_barrier(0);
        group_step<B, 1, FULL>(wb, sm.xs[(g + 3) % kRing], lane, nmt, tot);
        wait_and_sync<2 * kDmaOps + kLoadWOps<B>>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may land after the workgroup ends
}

}  // namespace

// Kernel modes: a plain layer, the same with outliers, or routed experts with one of the three
// grouped epilogues.
enum { kPlain = 0, kOutl = 1, kGroupNone = 2, kGroupSwiglu = 3, kGroupRowsF32 = 4 };

// FULL: every workgroup's eight 16-row activation tiles hold rows (a launch over whole
// 128-row tiles); otherwise tiles past the workgroup's rows are skipped.  mtile0: the first
// 128-row tile of the launch (plain layer).
template <int B, int MODE, bool FULL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(GemmArgs a,
                                                                                            int64_t mtile0,
                                                                                            int64_t m_tiles)
{
    constexpr bool OUTL = MODE == kOutl, GROUPED = MODE >= kGroupNone;
    __shared__ __attribute__((aligned(16))) Smem sm;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;
    const int64_t n_tiles = (a.n + kNT - 1) / kNT;
    int64_t nt, m0, mend;  // weight tile; sorted rows [m0, mend) of this workgroup
    int e = 0;
    if constexpr (GROUPED) {
        // blockIdx = (weight tile, expert, 128-row tile of the expert's rows)
        e = blockIdx.y;
        const int64_t r0 = a.offsets[e], r1 = a.offsets[e + 1];
        nt = blockIdx.x;
        m0 = r0 + (int64_t)blockIdx.z * kMRows;
        if (m0 >= r1) return;  // the whole workgroup: this expert has fewer row tiles
        mend = r1 < m0 + kMRows ? r1 : m0 + kMRows;
    } else {
        int64_t mtile;
        const int64_t b = blockIdx.x;
        if (n_tiles % 8 == 0) {  // XCD-aware: the m blocks of one n tile share an XCD
            const int64_t xcd = b % 8, local = b / 8;
            nt = (local / m_tiles) * 8 + xcd;
            mtile = local % m_tiles;
        } else {
            nt = b % n_tiles;
            mtile = b / n_tiles;
        }
        m0 = (mtile0 + mtile) * kMRows;
        mend = a.m < m0 + kMRows ? a.m : m0 + kMRows;
    }
    // 16-row activation tiles holding rows (uniform; tiles past it are skipped)
    const int nmt = (int)((mend - m0 + 15) / 16);
    const ExpertPtrs &W = a.ex[e];
    const int64_t NB = a.n / kTileN;
    const int64_t rb0 = nt * (kNT / kTileN) + wv * kRBW;  // first row block of this wave

    Bufs bf;
    // Activation rows are gathered per lane: the DMA source of a row past the workgroup's
    // rows lies past the buffer's range and reads zeros.
    bf.x = make_rsrc(a.x, a.m * a.ldx * 2);
#pragma unroll
    for (int it = 0; it < kDmaOps; ++it) {
        const int row = 16 * wv + 4 * it + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        const int64_t sr = m0 + row;
        int64_t src = sr;
        if constexpr (GROUPED) src = sr < mend ? (a.row_src ? a.row_src[sr] : sr) : 0;
        bf.xoff[it] = sr < mend ? (uint32_t)((src * a.ldx + 8 * c) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        const bool in = rb < NB;
        bf.w[u] = make_rsrc(W.packed + rb * KT * (512 * B), in ? KT * (512 * B) : 0);
        bf.sc[u] = make_rsrc(W.scales + rb * kTileN * G, in ? kTileN * G * 2 : 0);
        bf.zr[u] = make_rsrc(W.zeros + rb * kTileN * G, in ? kTileN * G : 0);
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

    k_loop<B, FULL>(bf, sm, KT, G, wv, lane, nmt, tot);

    // epilogue
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        if (rb >= NB) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int64_t row = m0 + 16 * mt + r;
            if (row >= mend) continue;
            const f4 s = tot[u][mt];
            if constexpr (MODE == kGroupRowsF32) {
                *(f4 *)((float *)a.y + row * a.ldy + rb * kTileN + 4 * t) = s;
            } else if constexpr (MODE == kGroupSwiglu) {
                // row blocks 2i (gate) and 2i+1 (up) of a wave: output features 16i + 4t + j
                if (u == 1) {
                    const f4 gt = tot[0][mt];
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = gt[j] / (1.0f + expf(-gt[j])) * s[j];
                    uint16_t *y = (uint16_t *)a.y + row * a.ldy + (rb / 2) * kTileN + 4 * t;
                    *(u2 *)y = (u2){pack_h2(o[0], o[1]), pack_h2(o[2], o[3])};
                }
            } else {
                uint16_t *y = (uint16_t *)a.y + row * a.ldy + rb * kTileN + 4 * t;
                *(u2 *)y = (u2){pack_h2(s[0], s[1]), pack_h2(s[2], s[3])};
            }
        }
    }
}

// x^T for the outlier partial: xt[kk][128 mb + 8 r + mt] = x[128 mb + 16 mt + r][kk], zeros
// for rows >= m.  One block per 64 k x 128 m tile: 16-byte loads of x rows into LDS, then
// each thread gathers eight values (one per tile mt) for one 16-byte store of x^T.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                                                        uint16_t *xt, int64_t ldxt)
{
    constexpr int kPitch = 64 + 2;  // halves per LDS row (odd dword pitch: rows hit distinct banks)
    __shared__ uint16_t tile[128 * kPitch];
    const int64_t k0 = blockIdx.x * 64, m0 = blockIdx.y * 128;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + 256 * it, row = idx / 8, c = idx % 8;
        const int64_t gm = m0 + row, gk = k0 + 8 * c;
        u4 v = {0u, 0u, 0u, 0u};
        if (gm < m && gk < k) v = *(const u4 *)(x + gm * ldx + gk);
        uint32_t *dst = (uint32_t *)(tile + row * kPitch + 8 * c);  // 4-byte aligned: kPitch even
        dst[0] = v[0];
        dst[1] = v[1];
        dst[2] = v[2];
        dst[3] = v[3];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + 256 * it, kk = idx / 16, sgm = idx % 16;  // positions 8 sgm ..
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            w[h] = (uint32_t)tile[(16 * (2 * h) + sgm) * kPitch + kk] |
                   ((uint32_t)tile[(16 * (2 * h + 1) + sgm) * kPitch + kk] << 16);
        const int64_t gk = k0 + kk;
        if (gk < k) *(u4 *)(xt + gk * ldxt + m0 + 8 * sgm) = (u4){w[0], w[1], w[2], w[3]};
    }
}

// Outlier partial: S^T[n][p] = sum over the outliers (n, c, v) of v * x^T[c][p], in fp32 (one
// wave per weight row, each lane 8 consecutive positions p of a 512-position chunk).  Eight
// entries are gathered per step so their loads are in flight together.
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
    for (int64_t e = e0; e < e1; e += 8) {
        u4 xv[8];
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = e + j < e1;
            v[j] = ok ? h_f(val[e + j]) : 0.f;
            xv[j] = ok ? *(const u4 *)(xt + (int64_t)col[e + j] * ldxt + p) : (u4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(lo_h(xv[j][q]), v[j], acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(hi_h(xv[j][q]), v[j], acc[2 * q + 1]);
            }
    }
    f4 *dst = (f4 *)(spart + row * ldxt + p);
    dst[0] = (f4){acc[0], acc[1], acc[2], acc[3]};
    dst[1] = (f4){acc[4], acc[5], acc[6], acc[7]};
}

// Whole 128-row tiles in one launch, a ragged last tile in another.
template <int B, int MODE>
static void gemm_launch(const GemmArgs &a, hipStream_t st)
{
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, full = a.m / kMRows;
    const dim3 block(kWaves * 64);
    if (full > 0)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, true>), dim3((unsigned)(n_tiles * full)), block, 0, st, a,
                           (int64_t)0, full);
    if (a.m % kMRows)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, false>), dim3((unsigned)n_tiles), block, 0, st, a, full, (int64_t)1);
}

template <int B>
static hipError_t gemm_bits(const GemmArgs &a, hipStream_t st)
{
    if (a.rowptr) {
        hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((a.k + 63) / 64), (unsigned)(a.ldxt / 128)), dim3(256), 0,
                           st, a.x, a.ldx, a.m, a.k, a.xt, a.ldxt);
        hipLaunchKernelGGL(outlier_spmm_kernel, dim3((unsigned)((a.n + 3) / 4), (unsigned)((a.ldxt + 511) / 512)),
                           dim3(256), 0, st, a.rowptr, a.col, a.val, a.xt, a.n, a.ldxt, a.spart);
        gemm_launch<B, kOutl>(a, st);
    } else {
        gemm_launch<B, kPlain>(a, st);
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

// Routed experts: one workgroup per (256-row weight tile, expert, 128-row tile of the
// expert's sorted rows); the row tiles are sized for the worst case (all rows on one expert)
// and the surplus workgroups return at once.
template <int B, int MODE>
static hipError_t grouped_mode(int n_experts, const GemmArgs &a, hipStream_t st)
{
    const int64_t n_tiles = (a.n + kNT - 1) / kNT, m_tiles = (a.m + kMRows - 1) / kMRows;
    hipLaunchKernelGGL((gemm_kernel<B, MODE, false>), dim3((unsigned)n_tiles, (unsigned)n_experts, (unsigned)m_tiles),
                       dim3(kWaves * 64), 0, st, a, (int64_t)0, m_tiles);
    return hipGetLastError();
}

template <int B>
static hipError_t grouped_bits(int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    switch (epilogue) {
    case QP_EPI_NONE: return grouped_mode<B, kGroupNone>(n_experts, a, st);
    case QP_EPI_SWIGLU: return grouped_mode<B, kGroupSwiglu>(n_experts, a, st);
    case QP_EPI_ROWS_F32: return grouped_mode<B, kGroupRowsF32>(n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(int bits, int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    if (a.m < 1) return hipSuccess;
    switch (bits) {
    case 2: return grouped_bits<2>(epilogue, n_experts, a, st);
    case 3: return grouped_bits<3>(epilogue, n_experts, a, st);
    case 4: return grouped_bits<4>(epilogue, n_experts, a, st);
    case 5: return grouped_bits<5>(epilogue, n_experts, a, st);
    case 6: return grouped_bits<6>(epilogue, n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qp
