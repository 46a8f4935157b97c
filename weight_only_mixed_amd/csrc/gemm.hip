// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  On CDNA4 the work is split
// differently.  Each of the eight waves of a workgroup owns two 16-row weight blocks and
// unpacks them itself into exact fp16 (q - zp) matrix-core A operands held in registers, so
// each weight is unpacked once per 128 activation rows and no unpacked weight passes through
// LDS.  The packed tiles are staged HBM -> LDS by buffer-to-LDS DMA two k-tiles ahead, each
// wave into its own part of a two-slot ring (no registers, no barrier).  The activation tile
// (128 rows x one 128-k group, 32 KB) is shared by the eight waves (256 weight rows) through
// a two-slot LDS ring filled by DMA one group ahead, its 16-byte chunks XOR-swizzled by row so
// the fragment reads (16 rows, same column) hit distinct banks.
//
// The k loop is software-pipelined across groups: while the matrix cores multiply group g,
// the vector ALU unpacks group g+1 and applies group g's scales, tile by tile, with the
// scheduler told to interleave one MFMA, one fragment read and two vector ops, so every wave
// keeps both units busy; the step's loads for later steps are issued a few per tile.  Every
// 128-k group is accumulated on the matrix cores in fp32 and then scaled by its fp16 scale in
// fp32 (mixed-bit page, s4.2).
//
// Routed experts (on-device MoE page, s4.2) run the same kernel on their sorted token rows.
// With few rows per expert a step is short and a wave's work in it mostly serial, so they use
// a smaller workgroup (four waves, 32 activation rows) of which three fit on a CU.
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
#include <algorithm>
#include <utility>

#include "unpack.h"
#include "wstage.h"

namespace qp {

namespace {

using namespace mm;

constexpr int kRowBytes = 128 * 2;  // one 128-k group of one activation row

// Workgroup geometry: W waves (2W weight row blocks) times MT 16-row activation tiles.
//  - Geo<8, 8>: 256 weight rows x 128 activation rows, one workgroup per CU (128 KB of LDS at
//    4 bits); the layer GEMM.
//  - Geo<4, 2>: 128 weight rows x 32 activation rows, three workgroups per CU (48 KB); routed
//    experts with few rows each, whose steps are too short to hide their latencies with two
//    waves per SIMD.
// Each wave stages kDmaX 1 KB runs of every activation slot (four rows each): rows
// 4 kDmaX wv .. 4 kDmaX (wv + 1) - 1.
template <int W, int MT>
struct Geo {
    static constexpr int kWaves = W;
    static constexpr int kMT = MT;
    static constexpr int kNT = W * kRBW * kTileN;    // weight rows per workgroup
    static constexpr int kMRows = MT * 16;           // activation rows per workgroup
    static constexpr int kXSlot = kMRows * kRowBytes;  // one activation slot
    static constexpr int kDmaX = kXSlot / 1024 / W;  // activation DMA instructions per wave per group
    static constexpr int kWavesPerEU = W == 8 ? 2 : 3;
    static_assert(kDmaX * 1024 * W == kXSlot && kDmaX >= 1, "whole 1 KB runs per wave");
};
using GeoLayer = Geo<8, 8>;
using GeoExperts = Geo<4, 2>;
static_assert(GeoLayer::kDmaX <= kDmaXMax && GeoExperts::kDmaX <= kDmaXMax, "activation DMA pieces per wave");

// LDS byte offset of 16-byte chunk c (8 k values) of activation row `row`.
__device__ __forceinline__ int xs_off(int row, int c) { return row * kRowBytes + ((c ^ (row & 15)) << 4); }

// Shared memory of one workgroup: a two-slot activation ring (one 128-k group per slot) and
// a two-slot ring of packed weight tiles (one k-tile per slot; every wave owns its part).
template <int B, typename G>
struct Smem {
    uint8_t xs[2][G::kXSlot];
    uint8_t ws[2][G::kWaves * kRBW * WStage<B>::kBytes];
};

// DMA the activation tile of group g (kMRows rows x 128 k) into LDS slot `dst` (this wave's
// kDmaX KB).  Lane L of piece `it` fills LDS bytes [16L, 16L+16) of a 1 KB run = row
// 4*(kDmaX*wv+it) + L/16, physical chunk L%16, which holds logical chunk (L%16) ^ (row & 15).
// When the workgroup's rows end before this wave's first row, its rows are never read and the
// wave issues nothing (out-of-range loads read zeros but still cost address-unit cycles).
template <typename G>
__device__ __forceinline__ bool stages_rows(int wv, int nmt)
{
    return 4 * G::kDmaX * wv < 16 * nmt;
}
template <typename G>
__device__ __forceinline__ void dma_x(const Bufs &bf, int64_t g, uint8_t *dst, int wv, int nmt)
{
    if (!stages_rows<G>(wv, nmt)) return;  // uniform
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)g * 256);  // column of group g
#pragma unroll
    for (int it = 0; it < G::kDmaX; ++it) lds_dma16(bf.x, dst + (wv * G::kDmaX + it) * 1024, bf.xoff[it], soff);
}

// Activation DMA piece `it` of this wave (four of its rows).
template <typename G>
__device__ __forceinline__ void dma_x_piece(const Bufs &bf, int64_t g, uint8_t *dst, int wv, int it)
{
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)g * 256);
    lds_dma16(bf.x, dst + (wv * G::kDmaX + it) * 1024, bf.xoff[it], soff);
}

// The share of a step's loads issued with activation tile MT of a full step: activation
// pieces with the first half of the tiles; scales and zero points with them too (even steps,
// so their memory latency has most of the step), the weight pieces with the second half (odd
// steps, after every activation piece, so the end-of-step wait can leave them in flight).
// Issuing everything at the start of a step instead stalls all eight waves together while
// the address unit works through about 48 KB.
template <int B, typename GE, int PAR, int NMT, int MT>
__device__ __forceinline__ void issue_tile(const Bufs &bf, const StepIO<PAR> &io, int64_t G, int wv, int lane)
{
    static_assert(NMT == GE::kMT && GE::kDmaX == NMT / 2, "one activation piece per tile of the first half");
    if constexpr (MT < NMT / 2) dma_x_piece<GE>(bf, io.gx, io.xdst, wv, MT);
    if constexpr (PAR == 0 && MT < NMT / 2) {
#pragma unroll
        for (int p = MT * kSZOps / (NMT / 2); p < (MT + 1) * kSZOps / (NMT / 2); ++p) load_sz_piece(bf, G, io.kt, lane, *io.z, p);
    }
    if constexpr (PAR == 1 && MT >= NMT / 2) {
        constexpr int q = MT - NMT / 2, h = NMT / 2;
#pragma unroll
        for (int p = q * kWOps<B> / h; p < (q + 1) * kWOps<B> / h; ++p) dma_w_piece<B>(bf, io.kt, io.wdst, lane, p);
    }
}

// All of a step's loads at once (ragged steps, whose tile count is not known at compile time).
template <int B, typename GE, int PAR>
__device__ __forceinline__ void issue_all(const Bufs &bf, const StepIO<PAR> &io, int64_t G, int wv, int lane, int nmt)
{
    dma_x<GE>(bf, io.gx, io.xdst, wv, nmt);
    if constexpr (PAR == 0) load_sz(bf, G, io.kt, lane, *io.z);
    else dma_w<B>(bf, io.kt, io.wdst, lane);
}

template <int B>
__device__ __forceinline__ void set_gc(const SZ &z, int half, GroupConst<B> (&gc)[kRBW])
{
#pragma unroll
    for (int u = 0; u < kRBW; ++u) gc[u].set(half == 0 ? (z.zz[u] & 0xFF) : ((z.zz[u] >> 8) & 0xFF));
}

// Unpack block J of group half H (blocks 4H .. 4H+3 of the chunk) of row block U.
template <int B, int H, int U, int J>
__device__ __forceinline__ void unpack_block(const uint32_t *d, const GroupConst<B> (&gc)[kRBW], h8 (&A)[kRBW][4])
{
    A[U][J] = BlockUnpack<B, 4 * H + J>::run(d, gc[U]);
}

// All of one group's A operands (this wave's two row blocks) from a staged weight slot part.
template <int B, int H>
__device__ __forceinline__ void unpack_group(const uint8_t *wpart, const SZ &z, int lane, h8 (&A)[kRBW][4])
{
    GroupConst<B> gc[kRBW];
    set_gc<B>(z, H, gc);
    uint32_t d[2 * B];
    read_chunk<B>(wpart, lane, d);
    unpack_block<B, H, 0, 0>(d, gc, A);
    unpack_block<B, H, 0, 1>(d, gc, A);
    unpack_block<B, H, 0, 2>(d, gc, A);
    unpack_block<B, H, 0, 3>(d, gc, A);
    read_chunk<B>(wpart + WStage<B>::kBytes, lane, d);
    unpack_block<B, H, 1, 0>(d, gc, A);
    unpack_block<B, H, 1, 1>(d, gc, A);
    unpack_block<B, H, 1, 2>(d, gc, A);
    unpack_block<B, H, 1, 3>(d, gc, A);
}

// Matrix-core chains of activation tile MT (fragments X) for both row blocks.
__device__ __forceinline__ void tile_mma(const h8 (&A)[kRBW][4], const h8 (&X)[4], f4 (&acc)[kRBW])
{
#pragma unroll
    for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][0], X[0], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j4 = 1; j4 < 4; ++j4)
#pragma unroll
        for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(A[u][j4], X[j4], acc[u]);
}

// tot[.][mt] += s * acc (fp32; the scale is the fp16 half SH of each packed scale word).
template <int SH, int MTS>
__device__ __forceinline__ void scale_acc(const uint32_t (&sc)[kRBW][4], const f4 (&acc)[kRBW], f4 (&tot)[kRBW][MTS],
                                          int mt)
{
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            tot[u][mt][i] = __builtin_fmaf(SH == 0 ? lo_h(sc[u][i]) : hi_h(sc[u][i]), acc[u][i], tot[u][mt][i]);
        asm volatile("" : "+v"(tot[u][mt]));
    }
}

// Activation fragment reads run kXA tiles ahead of the matrix core (ring of kXR tiles).
constexpr int kXA = 2, kXR = kXA + 1;

// Unpack blocks [F, L) of the next group (block i = row block i / 4, block i % 4).
template <int B, int NH, int F, int L>
__device__ __forceinline__ void unpack_range(const uint32_t *d, const GroupConst<B> (&gc)[kRBW], h8 (&A)[kRBW][4])
{
    if constexpr (F < L) {
        unpack_block<B, NH, F / 4, F % 4>(d, gc, A);
        unpack_range<B, NH, F + 1, L>(d, gc, A);
    }
}

// One activation tile of a full step of NMT tiles: fragment reads of tile MT+kXA, the
// matrix-core chains of tile MT, the scale-accumulate of tile MT-1 and a share of the next
// group's unpack (its eight blocks spread evenly over the NMT tiles; row block 1's chunk is
// read at tile NMT/2), interleaved so every wave keeps its matrix core and vector ALU busy.
template <int B, typename GE, int SH, int NH, int NMT, int MT>
__device__ __forceinline__ void full_tile(const h8 (&Acur)[kRBW][4], h8 (&Anxt)[kRBW][4], const uint32_t (&sc)[kRBW][4],
                                          const GroupConst<B> (&gc)[kRBW], const uint8_t *xs, const uint8_t *wpart,
                                          int lane, uint32_t (&d)[2 * B], h8 (&X)[kXR][4], f4 (&acc)[2][kRBW],
                                          f4 (&tot)[kRBW][GE::kMT], const Bufs &bf, const StepIO<NH ^ 1> &io,
                                          int64_t G, int wv)
{
    static_assert(NMT % 2 == 0 && NMT <= GE::kMT, "even tile count");
    constexpr int cur = MT & 1, nxt = cur ^ 1;
    const int t = lane >> 4, r = lane & 15;
    issue_tile<B, GE, NH ^ 1, NMT, MT>(bf, io, G, wv, lane);
    if constexpr (MT + kXA < NMT) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
            X[(MT + kXA) % kXR][j4] = *(const h8 *)(xs + xs_off(16 * (MT + kXA) + r, 4 * j4 + t));
    }
    if constexpr (MT == 0) read_chunk<B>(wpart, lane, d);
    if constexpr (MT == NMT / 2) read_chunk<B>(wpart + WStage<B>::kBytes, lane, d);
    tile_mma(Acur, X[MT % kXR], acc[cur]);
    if constexpr (MT > 0) scale_acc<SH>(sc, acc[nxt], tot, MT - 1);
    unpack_range<B, NH, MT * 8 / NMT, (MT + 1) * 8 / NMT>(d, gc, Anxt);
    if constexpr (MT == NMT - 1) scale_acc<SH>(sc, acc[cur], tot, MT);
    // per matrix-core op: one fragment read and two vector ALU ops issued behind it
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int B, typename GE, int SH, int NH, int NMT, int... MT>
__device__ __forceinline__ void full_tiles(std::integer_sequence<int, MT...>, const h8 (&Acur)[kRBW][4],
                                           h8 (&Anxt)[kRBW][4], const uint32_t (&sc)[kRBW][4],
                                           const GroupConst<B> (&gc)[kRBW], const uint8_t *xs, const uint8_t *wpart,
                                           int lane, uint32_t (&d)[2 * B], h8 (&X)[kXR][4], f4 (&acc)[2][kRBW],
                                           f4 (&tot)[kRBW][GE::kMT], const Bufs &bf, const StepIO<NH ^ 1> &io,
                                           int64_t G, int wv)
{
    (full_tile<B, GE, SH, NH, NMT, MT>(Acur, Anxt, sc, gc, xs, wpart, lane, d, X, acc, tot, bf, io, G, wv), ...);
}

// One 128-k group step: A(g) = Acur times the activation tile of group g (slot xs), scale
// half SH of scale words sc; meanwhile A(g+1) is unpacked into Anxt from half NH of the
// staged tile wpart with zero points zn, and the loads io for later steps are issued (a step
// that unpacks a first group, NH = 0, is an odd step).  NMT > 0: the first NMT 16-row
// activation tiles all hold rows; NMT == 0: nmt tiles hold rows (ragged), the loads are
// issued at once and the next group is unpacked first.
template <int B, typename GE, int SH, int NH, int NMT>
__device__ __forceinline__ void group_step(const h8 (&Acur)[kRBW][4], h8 (&Anxt)[kRBW][4], const uint32_t (&sc)[kRBW][4],
                                           const SZ &zn, const uint8_t *xs, const uint8_t *wpart, int lane, int nmt,
                                           f4 (&tot)[kRBW][GE::kMT], const Bufs &bf, const StepIO<NH ^ 1> &io,
                                           int64_t G, int wv)
{
    const int t = lane >> 4, r = lane & 15;
    f4 acc[2][kRBW];
    if constexpr (NMT > 0) {
        h8 X[kXR][4];
#pragma unroll
        for (int mt = 0; mt < kXA; ++mt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) X[mt][j4] = *(const h8 *)(xs + xs_off(16 * mt + r, 4 * j4 + t));
        GroupConst<B> gc[kRBW];
        set_gc<B>(zn, NH, gc);
        uint32_t d[2 * B];
        __builtin_amdgcn_sched_barrier(0);
        full_tiles<B, GE, SH, NH, NMT>(std::make_integer_sequence<int, NMT>{}, Acur, Anxt, sc, gc, xs, wpart, lane, d,
                                       X, acc, tot, bf, io, G, wv);
    } else {
        issue_all<B, GE, NH ^ 1>(bf, io, G, wv, lane, nmt);
        __builtin_amdgcn_sched_barrier(0);
        // Every ragged step has a first tile: its matrix-core chains run interleaved with the
        // unpack of the next group (few tiles leave the vector ALU the larger share), while
        // the second tile's fragments are read (rows past the workgroup's read stale LDS
        // bytes that are never used).
        h8 X[2][4];
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) X[0][j4] = *(const h8 *)(xs + xs_off(r, 4 * j4 + t));
        if constexpr (GE::kMT > 1) {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) X[1][j4] = *(const h8 *)(xs + xs_off(16 + r, 4 * j4 + t));
        }
        tile_mma(Acur, X[0], acc[0]);
        unpack_group<B, NH>(wpart, zn, lane, Anxt);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nmt == 1) scale_acc<SH>(sc, acc[0], tot, 0);
#pragma unroll
        for (int mt = 1; mt < GE::kMT; ++mt) {
            if (mt >= nmt) break;  // uniform: tiles past the workgroup's rows are skipped
            const int cur = mt & 1, nxt = cur ^ 1;
            if (mt + 1 < GE::kMT && mt + 1 < nmt) {
                const int row = 16 * (mt + 1) + r;
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) X[nxt][j4] = *(const h8 *)(xs + xs_off(row, 4 * j4 + t));
            }
            __builtin_amdgcn_sched_barrier(0);
            tile_mma(Acur, X[cur], acc[cur]);
            scale_acc<SH>(sc, acc[nxt], tot, mt - 1);
            if (mt + 1 == nmt) scale_acc<SH>(sc, acc[cur], tot, mt);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The k loop of a workgroup.  Step g multiplies group g and unpacks group g+1.
//  - Activations: slot g % 2 holds group g; the DMA of group g+1 into the other slot is
//    issued during step g (its previous contents were read in step g-1, which ended with a
//    workgroup barrier) and waited for at the end of step g.
//  - Weights: slot t % 2 holds k-tile t (every wave stages and reads only its own part, so
//    no barrier is involved).  Tile t is read while unpacking groups 2t and 2t+1, in steps
//    2t-1 and 2t; the DMA of tile t+2 into slot t % 2 is issued during step 2t+1, after that
//    step's activation DMA, and waited for at the end of step 2t+2.
//  - Scales and zero points of tile t are loaded into registers during step 2t-2.
//  In a full step the loads are spread over its activation tiles (issue_tile); in a ragged
//  step they are issued at its start.  The waits are: vmcnt(0) after steps 2t, and
//  vmcnt(weight DMAs) after steps 2t+1.  Loads past the end are clamped to the last group or
//  tile and land in slots that are not read again; the A operands unpacked from them are
//  discarded.
template <int B, typename GE, int NMT>
//  The four slots reach the loop as restrict pointers: that tells the compiler that reads of
//  one slot never touch a DMA in flight into another.  Without it (slots at run-time offsets
//  in one array) it waits for every outstanding load, the weight DMA meant to run a step and a
//  half ahead included, before each read of the ring.
__device__ __forceinline__ void k_loop(const Bufs &bf, uint8_t *__restrict__ xs0, uint8_t *__restrict__ xs1,
                                       uint8_t *__restrict__ ws0, uint8_t *__restrict__ ws1, int64_t KT, int64_t G, int wv, int lane, int nmt,
                                       f4 (&tot)[kRBW][GE::kMT])
{
    const int64_t GN = 2 * KT;  // groups
    auto gclamp = [&](int64_t g) { return g < GN ? g : GN - 1; };
    auto tclamp = [&](int64_t t) { return t < KT ? t : KT - 1; };
    uint8_t *w0 = ws0 + wv * (kRBW * WStage<B>::kBytes);  // this wave's parts of the weight slots
    uint8_t *w1 = ws1 + wv * (kRBW * WStage<B>::kBytes);
    (void)sizeof(GE);
    SZ z0, z1;  // tiles of even / odd index
    h8 Aa[kRBW][4], Ab[kRBW][4];

    dma_x<GE>(bf, 0, xs0, wv, nmt);
    dma_w<B>(bf, 0, w0, lane);
    dma_w<B>(bf, tclamp(1), w1, lane);
    load_sz(bf, G, 0, lane, z0);
    wait_and_sync<0>();
    retired(z0, bf.zmid);
    unpack_group<B, 0>(w0, z0, lane, Aa);

    for (int64_t kt = 0; kt < KT; kt += 2) {
        const int64_t g = 2 * kt;
        // step g: tile kt, first group; unpack tile kt's second group
        const StepIO<0> s0{gclamp(g + 1), tclamp(kt + 1), xs1, nullptr, &z1};
        group_step<B, GE, 0, 1, NMT>(Aa, Ab, z0.sc, z0, xs0, w0, lane, nmt, tot, bf, s0, G, wv);
        wait_and_sync<0>();
        retired(z1, bf.zmid);
        // step g+1: tile kt, second group; unpack tile kt+1's first group
        const StepIO<1> s1{gclamp(g + 2), tclamp(kt + 2), xs0, w0, nullptr};
        group_step<B, GE, 1, 0, NMT>(Ab, Aa, z0.sc, z1, xs1, w1, lane, nmt, tot, bf, s1, G, wv);
        wait_and_sync<kWOps<B>>();
        if (kt + 1 >= KT) break;
        // step g+2: tile kt+1, first group; unpack its second group
        const StepIO<0> s2{gclamp(g + 3), tclamp(kt + 2), xs1, nullptr, &z0};
        group_step<B, GE, 0, 1, NMT>(Aa, Ab, z1.sc, z1, xs0, w1, lane, nmt, tot, bf, s2, G, wv);
        wait_and_sync<0>();
        retired(z0, bf.zmid);
        // step g+3: tile kt+1, second group; unpack tile kt+2's first group
        const StepIO<1> s3{gclamp(g + 4), tclamp(kt + 3), xs0, w1, nullptr};
        group_step<B, GE, 1, 0, NMT>(Ab, Aa, z1.sc, z0, xs1, w0, lane, nmt, tot, bf, s3, G, wv);
        wait_and_sync<kWOps<B>>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may land after the workgroup ends
}

}  // namespace

// Kernel modes: a plain layer, the same with outliers, or routed experts with one of the three
// grouped epilogues.
enum { kPlain = 0, kOutl = 1, kGroupNone = 2, kGroupSwiglu = 3, kGroupRowsF32 = 4 };

// Workgroup -> (weight tile, activation rows) of a plain layer: up to two rectangles of
// weight tiles [nt0, nt0 + nnt) x activation tiles of mh rows starting at row m0, numbered
// from workgroup wg0 on.  Where nnt and wg0 are multiples of 8, the activation tiles of one
// weight tile get workgroups with equal index mod 8, which the dispatcher places on the same
// XCD, so they share its L2 copy of the packed weights.
struct TileRect {
    int32_t nt0, nnt, m0, mtiles, wg0;
};
struct TilePlan {
    TileRect r[2];
    int32_t nr;
    int32_t mh;       // activation rows per tile
    int32_t experts;  // grouped: entries of the offsets table, minus one
};

__device__ __forceinline__ void plan_tile(const TilePlan &p, int64_t b, int64_t &nt, int64_t &m0)
{
    const TileRect &R = (p.nr > 1 && b >= p.r[1].wg0) ? p.r[1] : p.r[0];
    const int64_t local = b - R.wg0;
    int64_t ntl, mt;
    if (R.nnt % 8 == 0 && R.wg0 % 8 == 0) {
        const int64_t xcd = local % 8, l8 = local / 8;
        ntl = (l8 / R.mtiles) * 8 + xcd;
        mt = l8 % R.mtiles;
    } else {
        ntl = local % R.nnt;
        mt = local / R.nnt;
    }
    nt = R.nt0 + ntl;
    m0 = R.m0 + mt * p.mh;
}

// NMT > 0: every workgroup's first NMT 16-row activation tiles hold rows; NMT == 0: a ragged
// workgroup (the last activation rows of a layer, or an expert's rows), tiles past its rows
// are skipped.
template <int B, int MODE, int NMT, typename GE>
__global__ __launch_bounds__(GE::kWaves * 64) __attribute__((amdgpu_waves_per_eu(GE::kWavesPerEU, GE::kWavesPerEU))) void gemm_kernel(
    GemmArgs a, TilePlan plan)
{
    constexpr bool OUTL = MODE == kOutl, GROUPED = MODE >= kGroupNone;
    constexpr int kMT = GE::kMT, kMRows = GE::kMRows;
    __shared__ __attribute__((aligned(16))) Smem<B, GE> sm;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / kGroup;
    // k range: all of k, or part blockIdx.z of a.ksplit equal parts (grouped fp32 rows)
    int64_t kt0 = 0, KTp = KT;
    if constexpr (MODE == kGroupRowsF32) {
        if (a.ksplit > 1) {
            KTp = KT / a.ksplit;
            kt0 = (int64_t)blockIdx.z * KTp;
        }
    }
    int64_t nt, m0, mend;  // weight tile; sorted rows [m0, mend) of this workgroup
    int e = 0;
    if constexpr (GROUPED) {
        // blockIdx = (weight tile, work item).  Work items number the occupied kMRows-row
        // tiles of all experts in expert order; lane i of every wave takes expert i's tile
        // count, a wave scan gives each expert its first work item, and the expert whose
        // range holds blockIdx.y serves this workgroup.  Surplus items return at once.
        const int32_t w = (int32_t)blockIdx.y;
        int32_t tiles = 0;
        if (lane < plan.experts) {
            const int32_t c = a.offsets[lane + 1] - a.offsets[lane];
            tiles = c > 0 ? (c + kMRows - 1) / kMRows : 0;
        }
        int32_t incl = tiles;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        const uint64_t hit = __ballot(lane < plan.experts && w >= incl - tiles && w < incl);
        if (!hit) return;  // the whole workgroup
        e = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
        const int32_t first = __shfl(incl - tiles, e);
        const int64_t r1 = a.offsets[e + 1];
        nt = blockIdx.x;
        m0 = a.offsets[e] + (int64_t)(w - first) * kMRows;
        mend = r1 < m0 + kMRows ? r1 : m0 + kMRows;
    } else {
        plan_tile(plan, blockIdx.x, nt, m0);
        mend = a.m < m0 + plan.mh ? a.m : m0 + plan.mh;
    }
    // 16-row activation tiles holding rows (uniform; tiles past it are skipped)
    const int nmt = (int)((mend - m0 + 15) / 16);
    const ExpertPtrs &W = a.ex[e];
    const int64_t NB = a.n / kTileN;
    const int64_t rb0 = nt * (GE::kNT / kTileN) + wv * kRBW;  // first row block of this wave

    Bufs bf;
    bf.zmid = a.zmid;
    // Activation rows are gathered per lane: the DMA source of a row past the workgroup's
    // rows lies past the buffer's range and reads zeros.
    bf.x = make_rsrc(a.x + kt0 * kTileK, (a.m * a.ldx - kt0 * kTileK) * 2);
#pragma unroll
    for (int it = 0; it < GE::kDmaX; ++it) {
        const int row = 4 * (GE::kDmaX * wv + it) + (lane >> 4);
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
        // tiles kt0 .. kt0 + KTp - 1 of the block; scale / zero point rows keep their stride G
        bf.w[u] = make_rsrc(W.packed + (rb * KT + kt0) * (512 * B), in ? KTp * (512 * B) : 0);
        bf.sc[u] = make_rsrc(W.scales + rb * kTileN * G + 2 * kt0, in ? (kTileN * G - 2 * kt0) * 2 : 0);
        bf.zr[u] = make_rsrc(W.zeros + rb * kTileN * G + 2 * kt0, in && !a.zmid ? kTileN * G - 2 * kt0 : 0);
    }

    f4 tot[kRBW][kMT];
    if constexpr (OUTL) {
        static_assert(kMT == 8, "the outlier partial's layout holds eight tiles per position block");
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

    k_loop<B, GE, NMT>(bf, sm.xs[0], sm.xs[1], sm.ws[0], sm.ws[1], KTp, G, wv, lane, nmt, tot);

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
                *(f4 *)((float *)a.y + (int64_t)blockIdx.z * a.ysplit + row * a.ldy + rb * kTileN + 4 * t) = s;
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

static TilePlan one_rect(int32_t nt0, int32_t nnt, int32_t m0, int32_t mtiles, int32_t mh)
{
    TilePlan p{};
    p.r[0] = {nt0, nnt, m0, mtiles, 0};
    p.nr = 1;
    p.mh = mh;
    return p;
}

// Whole 128-row activation tiles in one launch, a ragged last tile in another.
template <int B, int MODE>
static void gemm_launch(const GemmArgs &a, hipStream_t st)
{
    using GE = GeoLayer;
    const int32_t NT = (int32_t)((a.n + GE::kNT - 1) / GE::kNT), F = (int32_t)(a.m / GE::kMRows);
    const dim3 block(GE::kWaves * 64);
    if (F > 0)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, GE::kMT, GE>), dim3((unsigned)((int64_t)NT * F)), block, 0, st, a,
                           one_rect(0, NT, 0, F, GE::kMRows));
    if (a.m % GE::kMRows)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, 0, GE>), dim3((unsigned)NT), block, 0, st, a,
                           one_rect(0, NT, F * GE::kMRows, 1, GE::kMRows));
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

int64_t gemm_xt_ld(int64_t m) { return (m + GeoLayer::kMRows - 1) / GeoLayer::kMRows * GeoLayer::kMRows; }

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

// Routed experts: one workgroup per (weight tile, occupied row tile of an expert's sorted
// rows).  The row counts live on the device, so the grid holds the most row tiles any routing
// of a.m rows over the experts can occupy, sum over e of ceil(c_e / T) <= (a.m + E (T - 1)) / T,
// and the surplus workgroups return at once.  With at most 32 rows per expert on average the
// small geometry runs (three 4-wave workgroups per CU instead of one 8-wave one), else the
// layer's.
template <int B, int MODE, typename GE>
static hipError_t grouped_geo(int n_experts, const GemmArgs &a, hipStream_t st)
{
    constexpr int64_t T = GE::kMRows;
    const int64_t n_tiles = (a.n + GE::kNT - 1) / GE::kNT;
    const int64_t items = std::min<int64_t>((a.m + n_experts * (T - 1)) / T, n_experts * ((a.m + T - 1) / T));
    TilePlan plan{};
    plan.experts = n_experts;
    const unsigned parts = MODE == kGroupRowsF32 && a.ksplit > 1 ? (unsigned)a.ksplit : 1u;
    hipLaunchKernelGGL((gemm_kernel<B, MODE, 0, GE>), dim3((unsigned)n_tiles, (unsigned)items, parts),
                       dim3(GE::kWaves * 64), 0, st, a, plan);
    return hipGetLastError();
}
template <int B, int MODE>
static hipError_t grouped_mode(int n_experts, const GemmArgs &a, hipStream_t st)
{
    if (a.m <= (int64_t)GeoExperts::kMRows * n_experts) return grouped_geo<B, MODE, GeoExperts>(n_experts, a, st);
    return grouped_geo<B, MODE, GeoLayer>(n_experts, a, st);
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
