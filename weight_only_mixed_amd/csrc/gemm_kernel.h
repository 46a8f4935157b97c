// Prefill dequant-GEMM (m >= 64) on gfx950 matrix cores: the kernel templates, instantiated
// per group size and zero-point form in gemm.hip, gemm_g64.hip, gemm_g32.hip and gemm_zp.hip.
//
// Prior art: the fused dequant-GEMM of the single-GPU 70B page (s3) loads an INT4 tile into
// shared memory, dequantizes it and feeds Tensor Cores.  On CDNA4 the work is split
// differently.  Each of the eight waves of a workgroup owns two 16-row weight blocks and
// unpacks them itself into exact fp16 (q - zp) matrix-core operands held in registers, so
// each weight is unpacked once per 128 activation rows and no unpacked weight passes through
// LDS.  The packed tiles are staged HBM -> LDS by buffer-to-LDS DMA two k-tiles ahead, each
// wave into its own part of a two-slot ring (no registers, no barrier).  The activation tile
// (128 rows x one 128-k group, 32 KB) is shared by the eight waves (256 weight rows) through
// a two-slot LDS ring filled by DMA one group ahead, its 16-byte chunks XOR-swizzled by row so
// the fragment reads (16 rows, same column) hit distinct banks.
//
// The activations are the matrix core's A operand and the weights its B operand: a lane's four
// results are four activation rows of one weight row, so it needs one scale and one zero point
// per group (groups of 32, 64 or 128; mixed-bit page, s2.3).  Each 128-k step runs as units
// (16-row activation tile, group): a group's products are accumulated on the matrix cores in
// fp32 and then scaled by its fp16 scale in fp32 (mixed-bit page, s4.2) right after the next
// unit's matrix-core ops are issued.
//
// The k loop is software-pipelined across steps: while the matrix cores multiply step g, the
// vector ALU unpacks step g+1 and applies step g's scales, tile by tile, with the scheduler
// told to interleave one MFMA, one fragment read and two vector ops, so every wave keeps both
// units busy; the step's loads for later steps are issued a few per tile.  Zero points stored
// in b bits (ZPK) are expanded to bytes in registers when their loads retire.
//
// Routed experts (on-device MoE page, s4.2) run the same kernel on their sorted token rows.
// With few rows per expert a step is short and a wave's work in it mostly serial, so they use
// a smaller workgroup (four waves, 32 activation rows) of which three fit on a CU.
//
// Outlier add-back (70B page, s2): the held-out fp16 weights are added in fp32 before the one
// fp16 rounding of y.  Two small kernels run first (gemm.hip): one writes x transposed (x^T)
// into the caller's workspace, the other multiplies each weight row's outliers by it into an
// fp32 sparse partial S^T[n][m].  The GEMM then starts its fp32 accumulators from S^T instead
// of zero, so the main loop is the same as without outliers.  Inside each 128-row block of m
// the transposed layouts keep activation row 16 mt + 4 t + i at position 32 t + 4 mt + i: a
// lane's accumulators (tiles mt = 0..7, rows 4t + i) are 32 consecutive floats of S^T.
//
// Workgroups are ordered so that the activation blocks of one weight tile run on the same XCD
// (block b runs on XCD b % 8), where they share that XCD's L2 copy of the packed weights.
#pragma once

#include <algorithm>
#include <utility>

#include "unpack.h"
#include "wstage.h"

namespace qp {
namespace gk {

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
template <int B, typename GE, int GS, int ZPK, int PAR, int NMT, int MT>
__device__ __forceinline__ void issue_tile(const Bufs &bf, const StepIO<PAR, GS> &io, int64_t G, int wv, int lane)
{
    static_assert(NMT == GE::kMT && GE::kDmaX == NMT / 2, "one activation piece per tile of the first half");
    if constexpr (MT < NMT / 2) dma_x_piece<GE>(bf, io.gx, io.xdst, wv, MT);
    if constexpr (PAR == 0 && MT < NMT / 2) {
#pragma unroll
        for (int p = MT * kSZOps / (NMT / 2); p < (MT + 1) * kSZOps / (NMT / 2); ++p)
            load_sz_piece<B, GS, ZPK>(bf, G, io.kt, lane, *io.z, p);
    }
    if constexpr (PAR == 1 && MT >= NMT / 2) {
        constexpr int q = MT - NMT / 2, h = NMT / 2;
#pragma unroll
        for (int p = q * kWOps<B> / h; p < (q + 1) * kWOps<B> / h; ++p) dma_w_piece<B>(bf, io.kt, io.wdst, lane, p);
    }
}

// All of a step's loads at once (ragged steps, whose tile count is not known at compile time).
template <int B, typename GE, int GS, int ZPK, int PAR>
__device__ __forceinline__ void issue_all(const Bufs &bf, const StepIO<PAR, GS> &io, int64_t G, int wv, int lane,
                                          int nmt)
{
    dma_x<GE>(bf, io.gx, io.xdst, wv, nmt);
    if constexpr (PAR == 0) load_sz<B, GS, ZPK>(bf, G, io.kt, lane, *io.z);
    else dma_w<B>(bf, io.kt, io.wdst, lane);
}

// Groups per 128-k step (1, 2 or 4) and matrix-core ops (K = 32) per group.
template <int GS>
constexpr int kNGH = kGroup / GS;
template <int GS>
constexpr int kChain = 4 / kNGH<GS>;

// Bias constants of the unpack for group half H of a tile (groups of 128: one per row block,
// set once per step; smaller groups set theirs per block in unpack_block).
template <int B, int GS, int H>
__device__ __forceinline__ void set_gc(const SZ<GS> &z, GroupConst<B> (&gc)[kRBW])
{
    if constexpr (GS == kGroup) {
#pragma unroll
        for (int u = 0; u < kRBW; ++u) gc[u].set(zp_of(z, u, H));
    }
}

// Unpack block J of group half H (blocks 4H .. 4H+3 of the chunk) of row block U.  Block J
// covers k 32J .. 32J+31 of the half: group H * kNGH + J / kChain of the tile.
template <int B, int GS, int H, int U, int J>
__device__ __forceinline__ void unpack_block(const uint32_t *d, const SZ<GS> &z, const GroupConst<B> (&gc)[kRBW],
                                             h8 (&A)[kRBW][4])
{
    if constexpr (GS == kGroup) {
        A[U][J] = BlockUnpack<B, 4 * H + J>::run(d, gc[U]);
    } else {
        GroupConst<B> g;
        g.set(zp_of(z, U, H * kNGH<GS> + J / kChain<GS>));
        A[U][J] = BlockUnpack<B, 4 * H + J>::run(d, g);
    }
}

// All of one group's operands (this wave's two row blocks) from a staged weight slot part.
template <int B, int GS, int H>
__device__ __forceinline__ void unpack_group(const uint8_t *wpart, const SZ<GS> &z, int lane, h8 (&A)[kRBW][4])
{
    GroupConst<B> gc[kRBW];
    set_gc<B, GS, H>(z, gc);
    uint32_t d[2 * B];
    read_chunk<B>(wpart, lane, d);
    unpack_block<B, GS, H, 0, 0>(d, z, gc, A);
    unpack_block<B, GS, H, 0, 1>(d, z, gc, A);
    unpack_block<B, GS, H, 0, 2>(d, z, gc, A);
    unpack_block<B, GS, H, 0, 3>(d, z, gc, A);
    read_chunk<B>(wpart + WStage<B>::kBytes, lane, d);
    unpack_block<B, GS, H, 1, 0>(d, z, gc, A);
    unpack_block<B, GS, H, 1, 1>(d, z, gc, A);
    unpack_block<B, GS, H, 1, 2>(d, z, gc, A);
    unpack_block<B, GS, H, 1, 3>(d, z, gc, A);
}

// Matrix-core chain of group C of the step for activation tile fragments X, both row blocks.
// The activations are the A operand and the weights the B operand, so a lane's four results
// are four activation rows (4t + i) of one weight row (r): one scale per lane and group.
template <int GS, int C>
__device__ __forceinline__ void chain_mma(const h8 (&A)[kRBW][4], const h8 (&X)[4], f4 (&acc)[kRBW])
{
    constexpr int j0 = C * kChain<GS>;
#pragma unroll
    for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(X[j0], A[u][j0], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 1; j < kChain<GS>; ++j)
#pragma unroll
        for (int u = 0; u < kRBW; ++u) acc[u] = mfma16(X[j0 + j], A[u][j0 + j], acc[u]);
}
template <int GS, int... C>
__device__ __forceinline__ void chains_mma(std::integer_sequence<int, C...>, const h8 (&A)[kRBW][4], const h8 (&X)[4],
                                           f4 (&acc)[kNGH<GS>][kRBW])
{
    (chain_mma<GS, C>(A, X, acc[C]), ...);
}

// tot[.][mt] += s * acc for group q of the tile (fp32; s the fp16 scale of the lane's row).
template <int GS, int MTS>
__device__ __forceinline__ void scale_acc(const SZ<GS> &z, int q, const f4 (&acc)[kRBW], f4 (&tot)[kRBW][MTS], int mt)
{
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const float s = sc_of(z, u, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[u][mt][i] = __builtin_fmaf(s, acc[u][i], tot[u][mt][i]);
        asm volatile("" : "+v"(tot[u][mt]));
    }
}

// Activation fragment reads run kXA tiles ahead of the matrix core (ring of kXR tiles).
constexpr int kXA = 2, kXR = kXA + 1;

// Unpack blocks [F, L) of the next group (block i = row block i / 4, block i % 4).
template <int B, int GS, int NH, int F, int L>
__device__ __forceinline__ void unpack_range(const uint32_t *d, const SZ<GS> &z, const GroupConst<B> (&gc)[kRBW],
                                             h8 (&A)[kRBW][4])
{
    if constexpr (F < L) {
        unpack_block<B, GS, NH, F / 4, F % 4>(d, z, gc, A);
        unpack_range<B, GS, NH, F + 1, L>(d, z, gc, A);
    }
}

// The matrix-core work of a step is a sequence of units (tile mt, group c of the step), unit
// v = mt * kNGH + c.  Each unit's products are scaled into tot right after the next unit's
// matrix-core ops are issued (two accumulator sets, whatever the group size).
template <int GS, int SH, int MTS, int V>
__device__ __forceinline__ void scale_unit(const SZ<GS> &zs, const f4 (&acc)[2][kRBW], f4 (&tot)[kRBW][MTS])
{
    scale_acc<GS, MTS>(zs, SH * kNGH<GS> + V % kNGH<GS>, acc[V & 1], tot, V / kNGH<GS>);
}
template <int GS, int SH, int MTS, int MT, int C>
__device__ __forceinline__ void tile_unit(const h8 (&A)[kRBW][4], const h8 (&X)[4], const SZ<GS> &zs,
                                          f4 (&acc)[2][kRBW], f4 (&tot)[kRBW][MTS])
{
    constexpr int v = MT * kNGH<GS> + C;
    chain_mma<GS, C>(A, X, acc[v & 1]);
    if constexpr (v > 0) scale_unit<GS, SH, MTS, v - 1>(zs, acc, tot);
}
template <int GS, int SH, int MTS, int MT, int... C>
__device__ __forceinline__ void tile_units(std::integer_sequence<int, C...>, const h8 (&A)[kRBW][4], const h8 (&X)[4],
                                           const SZ<GS> &zs, f4 (&acc)[2][kRBW], f4 (&tot)[kRBW][MTS])
{
    (tile_unit<GS, SH, MTS, MT, C>(A, X, zs, acc, tot), ...);
}

// One activation tile of a full step of NMT tiles: fragment reads of tile MT+kXA, the
// matrix-core units of tile MT (each scaling the unit before it), and a share of the next
// group's unpack (its eight blocks spread evenly over the NMT tiles; row block 1's chunk is
// read at tile NMT/2), interleaved so every wave keeps its matrix core and vector ALU busy.
template <int B, typename GE, int GS, int ZPK, int SH, int NH, int NMT, int MT>
__device__ __forceinline__ void full_tile(const h8 (&Acur)[kRBW][4], h8 (&Anxt)[kRBW][4], const SZ<GS> &zs,
                                          const SZ<GS> &zn, const GroupConst<B> (&gc)[kRBW], const uint8_t *xs,
                                          const uint8_t *wpart, int lane, uint32_t (&d)[2 * B], h8 (&X)[kXR][4],
                                          f4 (&acc)[2][kRBW], f4 (&tot)[kRBW][GE::kMT], const Bufs &bf,
                                          const StepIO<NH ^ 1, GS> &io, int64_t G, int wv)
{
    static_assert(NMT % 2 == 0 && NMT <= GE::kMT, "even tile count");
    const int t = lane >> 4, r = lane & 15;
    issue_tile<B, GE, GS, ZPK, NH ^ 1, NMT, MT>(bf, io, G, wv, lane);
    if constexpr (MT + kXA < NMT) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
            X[(MT + kXA) % kXR][j4] = *(const h8 *)(xs + xs_off(16 * (MT + kXA) + r, 4 * j4 + t));
    }
    if constexpr (MT == 0) read_chunk<B>(wpart, lane, d);
    if constexpr (MT == NMT / 2) read_chunk<B>(wpart + WStage<B>::kBytes, lane, d);
    tile_units<GS, SH, GE::kMT, MT>(std::make_integer_sequence<int, kNGH<GS>>{}, Acur, X[MT % kXR], zs, acc, tot);
    unpack_range<B, GS, NH, MT * 8 / NMT, (MT + 1) * 8 / NMT>(d, zn, gc, Anxt);
    if constexpr (MT == NMT - 1) scale_unit<GS, SH, GE::kMT, NMT * kNGH<GS> - 1>(zs, acc, tot);
    // per matrix-core op: one fragment read and two vector ALU ops issued behind it
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int B, typename GE, int GS, int ZPK, int SH, int NH, int NMT, int... MT>
__device__ __forceinline__ void full_tiles(std::integer_sequence<int, MT...>, const h8 (&Acur)[kRBW][4],
                                           h8 (&Anxt)[kRBW][4], const SZ<GS> &zs, const SZ<GS> &zn,
                                           const GroupConst<B> (&gc)[kRBW], const uint8_t *xs, const uint8_t *wpart,
                                           int lane, uint32_t (&d)[2 * B], h8 (&X)[kXR][4], f4 (&acc)[2][kRBW],
                                           f4 (&tot)[kRBW][GE::kMT], const Bufs &bf, const StepIO<NH ^ 1, GS> &io,
                                           int64_t G, int wv)
{
    (full_tile<B, GE, GS, ZPK, SH, NH, NMT, MT>(Acur, Anxt, zs, zn, gc, xs, wpart, lane, d, X, acc, tot, bf, io, G, wv), ...);
}

// Ragged steps: the units of tile mt (the loop over tiles is unrolled, so mt and every
// accumulator index are compile-time after unrolling), each scaling the unit before it; the
// last tile (mt = nmt - 1) also scales its own last unit.
template <int GS, int SH, int MTS, int... C>
__device__ __forceinline__ void ragged_tile(std::integer_sequence<int, C...>, const h8 (&A)[kRBW][4],
                                            const h8 (&X)[4], const SZ<GS> &zs, f4 (&acc)[2][kRBW],
                                            f4 (&tot)[kRBW][MTS], int mt, int nmt)
{
    auto unit = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const int v = mt * kNGH<GS> + c;
        chain_mma<GS, c>(A, X, acc[v & 1]);
        if (v > 0) {
            const int pv = v - 1;
            scale_acc<GS, MTS>(zs, SH * kNGH<GS> + pv % kNGH<GS>, acc[pv & 1], tot, pv / kNGH<GS>);
        }
    };
    (unit(std::integral_constant<int, C>{}), ...);
    if (mt + 1 == nmt) {
        const int v = mt * kNGH<GS> + kNGH<GS> - 1;
        scale_acc<GS, MTS>(zs, SH * kNGH<GS> + kNGH<GS> - 1, acc[v & 1], tot, mt);
    }
}

// One 128-k group step: the step's weights Acur times the activation tile of group g (slot
// xs), scales of group half SH of tile metadata zs; meanwhile the next group is unpacked into
// Anxt from half NH of the staged tile wpart with metadata zn, and the loads io for later steps
// are issued (a step that unpacks a first group, NH = 0, is an odd step).  NMT > 0: the first
// NMT 16-row activation tiles all hold rows; NMT == 0: nmt tiles hold rows (ragged), the loads
// are issued at once and the next group is unpacked first.
template <int B, typename GE, int GS, int ZPK, int SH, int NH, int NMT>
__device__ __forceinline__ void group_step(const h8 (&Acur)[kRBW][4], h8 (&Anxt)[kRBW][4], const SZ<GS> &zs,
                                           const SZ<GS> &zn, const uint8_t *xs, const uint8_t *wpart, int lane,
                                           int nmt, f4 (&tot)[kRBW][GE::kMT], const Bufs &bf,
                                           const StepIO<NH ^ 1, GS> &io, int64_t G, int wv)
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
        set_gc<B, GS, NH>(zn, gc);
        uint32_t d[2 * B];
        __builtin_amdgcn_sched_barrier(0);
        full_tiles<B, GE, GS, ZPK, SH, NH, NMT>(std::make_integer_sequence<int, NMT>{}, Acur, Anxt, zs, zn, gc, xs, wpart,
                                           lane, d, X, acc, tot, bf, io, G, wv);
    } else {
        issue_all<B, GE, GS, ZPK, NH ^ 1>(bf, io, G, wv, lane, nmt);
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
        ragged_tile<GS, SH, GE::kMT>(std::make_integer_sequence<int, kNGH<GS>>{}, Acur, X[0], zs, acc, tot, 0, nmt);
        unpack_group<B, GS, NH>(wpart, zn, lane, Anxt);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
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
            ragged_tile<GS, SH, GE::kMT>(std::make_integer_sequence<int, kNGH<GS>>{}, Acur, X[cur], zs, acc, tot, mt, nmt);
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
template <int B, typename GE, int GS, int ZPK, int NMT>
//  The four slots reach the loop as restrict pointers: that tells the compiler that reads of
//  one slot never touch a DMA in flight into another.  Without it (slots at run-time offsets
//  in one array) it waits for every outstanding load, the weight DMA meant to run a step and a
//  half ahead included, before each read of the ring.
__device__ __forceinline__ void k_loop(const Bufs &bf, uint8_t *__restrict__ xs0, uint8_t *__restrict__ xs1,
                                       uint8_t *__restrict__ ws0, uint8_t *__restrict__ ws1, int64_t KT, int64_t G, int wv, int lane, int nmt,
                                       f4 (&tot)[kRBW][GE::kMT])
{
    const int64_t GN = 2 * KT;  // 128-k steps
    auto gclamp = [&](int64_t g) { return g < GN ? g : GN - 1; };
    auto tclamp = [&](int64_t t) { return t < KT ? t : KT - 1; };
    uint8_t *w0 = ws0 + wv * (kRBW * WStage<B>::kBytes);  // this wave's parts of the weight slots
    uint8_t *w1 = ws1 + wv * (kRBW * WStage<B>::kBytes);
    SZ<GS> z0{}, z1{};  // metadata of tiles of even / odd index
    h8 Aa[kRBW][4], Ab[kRBW][4];

    dma_x<GE>(bf, 0, xs0, wv, nmt);
    dma_w<B>(bf, 0, w0, lane);
    dma_w<B>(bf, tclamp(1), w1, lane);
    load_sz<B, GS, ZPK>(bf, G, 0, lane, z0);
    wait_and_sync<0>();
    retired<B, GS, ZPK>(z0, bf, 0);
    // Opaque accumulators from here on (whatever they start from: zeros, or the outlier
    // partial whose loads the wait above has also retired).  Known starting values let the
    // compiler specialise the first steps and spill; a barrier at the partial's loads would
    // make the prologue's DMA wait for them.
#pragma unroll
    for (int u = 0; u < kRBW; ++u)
#pragma unroll
        for (int mt = 0; mt < GE::kMT; ++mt) asm volatile("" : "+v"(tot[u][mt]));
    unpack_group<B, GS, 0>(w0, z0, lane, Aa);

    for (int64_t kt = 0; kt < KT; kt += 2) {
        const int64_t g = 2 * kt;
        // step g: tile kt, first group; unpack tile kt's second group
        const StepIO<0, GS> s0{gclamp(g + 1), tclamp(kt + 1), xs1, nullptr, &z1};
        group_step<B, GE, GS, ZPK, 0, 1, NMT>(Aa, Ab, z0, z0, xs0, w0, lane, nmt, tot, bf, s0, G, wv);
        wait_and_sync<0>();
        retired<B, GS, ZPK>(z1, bf, tclamp(kt + 1));
        // step g+1: tile kt, second group; unpack tile kt+1's first group
        const StepIO<1, GS> s1{gclamp(g + 2), tclamp(kt + 2), xs0, w0, nullptr};
        group_step<B, GE, GS, ZPK, 1, 0, NMT>(Ab, Aa, z0, z1, xs1, w1, lane, nmt, tot, bf, s1, G, wv);
        wait_and_sync<kWOps<B>>();
        if (kt + 1 >= KT) break;
        // step g+2: tile kt+1, first group; unpack its second group
        const StepIO<0, GS> s2{gclamp(g + 3), tclamp(kt + 2), xs1, nullptr, &z0};
        group_step<B, GE, GS, ZPK, 0, 1, NMT>(Aa, Ab, z1, z1, xs0, w1, lane, nmt, tot, bf, s2, G, wv);
        wait_and_sync<0>();
        retired<B, GS, ZPK>(z0, bf, tclamp(kt + 2));
        // step g+3: tile kt+1, second group; unpack tile kt+2's first group
        const StepIO<1, GS> s3{gclamp(g + 4), tclamp(kt + 3), xs0, w1, nullptr};
        group_step<B, GE, GS, ZPK, 1, 0, NMT>(Ab, Aa, z1, z0, xs1, w0, lane, nmt, tot, bf, s3, G, wv);
        wait_and_sync<kWOps<B>>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may land after the workgroup ends
}


// Kernel modes: a plain layer, the same with outliers, routed experts with one of the three
// grouped epilogues, or a plain layer split into k parts writing fp32 partial rows.
enum { kPlain = 0, kOutl = 1, kGroupNone = 2, kGroupSwiglu = 3, kGroupRowsF32 = 4, kSplitF32 = 5 };

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
// Both travel as kernel arguments: keep them within 4 KB.
static_assert(sizeof(GemmArgs) + sizeof(TilePlan) <= 4096, "kernel arguments over 4 KB");

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
template <int B, int MODE, int NMT, typename GE, int GS, int ZPK>
__global__ __launch_bounds__(GE::kWaves * 64) __attribute__((amdgpu_waves_per_eu(GE::kWavesPerEU, GE::kWavesPerEU))) void gemm_kernel(
    GemmArgs a, TilePlan plan)
{
    constexpr bool OUTL = MODE == kOutl, GROUPED = MODE >= kGroupNone && MODE <= kGroupRowsF32;
    constexpr bool KSPLIT = MODE == kGroupRowsF32 || MODE == kSplitF32;
    constexpr int kMT = GE::kMT, kMRows = GE::kMRows;
    __shared__ __attribute__((aligned(16))) Smem<B, GE> sm;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / GS;  // G: groups per weight row
    // k range: all of k, or part blockIdx.z of a.ksplit equal parts (fp32 rows)
    int64_t kt0 = 0, KTp = KT;
    if constexpr (KSPLIT) {
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
    bf.zrow = a.zrow;
    bf.kt0 = (uint32_t)kt0;
    bf.rowf = make_rsrc(W.rowf, W.rowf ? a.n * 4 : 0);
    bf.row0 = (uint32_t)(rb0 * kTileN);
    bf.fb = make_rsrc(W.fb, W.fb ? a.n * W.fb_stride * 2 : 0);
    bf.fbs = W.fb_stride;
    const int64_t zstride = a.zrow ? a.zrow : G;  // zero-point bytes per weight row
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
        // tiles kt0 .. kt0 + KTp - 1 of the block; scales and zero points are read from their
        // rows' starts (bf.kt0 offsets the tile index)
        bf.w[u] = make_rsrc(W.packed + (rb * KT + kt0) * (512 * B), in ? KTp * (512 * B) : 0);
        if constexpr (ZPK == kZpFp8)  // scale bytes
            bf.sc[u] = make_rsrc((const uint8_t *)W.scales + rb * kTileN * G, in ? kTileN * G : 0);
        else
            bf.sc[u] = make_rsrc(W.scales + rb * kTileN * G, in ? kTileN * G * 2 : 0);
        bf.zr[u] = make_rsrc(W.zeros + rb * kTileN * zstride, in && !a.zmid ? kTileN * zstride : 0);
    }

    f4 tot[kRBW][kMT];
    // the outlier partial seeds the accumulators of an outlier layer, and of the first k part
    // of a split one (the parts are summed afterwards)
    bool seed = false;
    if constexpr (OUTL) seed = true;
    if constexpr (MODE == kSplitF32) seed = blockIdx.z == 0 && a.spart != nullptr;
    if constexpr (OUTL || MODE == kSplitF32) {
        static_assert(kMT == 8, "the outlier partial's layout holds eight tiles per position block");
        if (seed) {
            // accumulators start from S^T (rows past n read as zeros): inside each 128-row
            // block, activation row 16 mt + 4 t + i sits at position 32 t + 4 mt + i, so a
            // lane's tot[u][0..7] are 32 consecutive floats of weight row rb * 16 + r
            const rsrc_t sr = make_rsrc(a.spart, a.n * a.ldxt * 4);
#pragma unroll
            for (int u = 0; u < kRBW; ++u) {
                const uint32_t off = (uint32_t)((((rb0 + u) * kTileN + r) * a.ldxt + m0 + 32 * t) * 4);
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    const u4 v = ld16(sr, off + 16 * mt);
                    tot[u][mt] = (f4){as_f(v[0]), as_f(v[1]), as_f(v[2]), as_f(v[3])};
                }
            }
        }
    }
    if (!seed) {
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

    k_loop<B, GE, GS, ZPK, NMT>(bf, sm.xs[0], sm.xs[1], sm.ws[0], sm.ws[1], KTp, G, wv, lane, nmt, tot);

    // epilogue: lane (t, r) holds, per row block u and tile mt, activation rows 16 mt + 4 t + i
    // of weight row rb * 16 + r (sixteen lanes store 16 consecutive outputs of a row)
    float rowf[kRBW];  // fp8 scales: each row block's weight-row factor (1 otherwise)
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        rowf[u] = 1.0f;
        if constexpr (ZPK == kZpFp8)
            if (rb0 + u < NB) rowf[u] = W.rowf[(rb0 + u) * kTileN + r];
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        if (rb >= NB) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + 16 * mt + 4 * t + i;
                if (row >= mend) continue;
                float v = tot[u][mt][i];
                if constexpr (ZPK == kZpFp8) v *= rowf[u];
                if constexpr (KSPLIT) {
                    ((float *)a.y)[(int64_t)blockIdx.z * a.ysplit + row * a.ldy + rb * kTileN + r] = v;
                } else if constexpr (MODE == kGroupSwiglu) {
                    // row blocks 2j (gate) and 2j+1 (up) of a wave: output feature 16 j + r
                    if (u == 1) {
                        float gt = tot[0][mt][i];
                        if constexpr (ZPK == kZpFp8) gt *= rowf[0];
                        const float o = gt / (1.0f + expf(-gt)) * v;
                        ((uint16_t *)a.y)[row * a.ldy + (rb / 2) * kTileN + r] = __builtin_bit_cast(uint16_t, (_Float16)o);
                    }
                } else {
                    ((uint16_t *)a.y)[row * a.ldy + rb * kTileN + r] = __builtin_bit_cast(uint16_t, (_Float16)v);
                }
            }
        }
    }
}

static inline TilePlan one_rect(int32_t nt0, int32_t nnt, int32_t m0, int32_t mtiles, int32_t mh)
{
    TilePlan p{};
    p.r[0] = {nt0, nnt, m0, mtiles, 0};
    p.nr = 1;
    p.mh = mh;
    return p;
}

// Whole 128-row activation tiles in one launch, a ragged last tile in another (kSplitF32: each
// with a.ksplit k parts as the grid's third dimension).
template <int B, int MODE, int GS, int ZPK>
void gemm_launch(const GemmArgs &a, hipStream_t st)
{
    using GE = GeoLayer;
    const int32_t NT = (int32_t)((a.n + GE::kNT - 1) / GE::kNT), F = (int32_t)(a.m / GE::kMRows);
    const unsigned parts = MODE == kSplitF32 ? (unsigned)a.ksplit : 1u;
    const dim3 block(GE::kWaves * 64);
    if (F > 0)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, GE::kMT, GE, GS, ZPK>), dim3((unsigned)((int64_t)NT * F), 1, parts),
                           block, 0, st, a, one_rect(0, NT, 0, F, GE::kMRows));
    if (a.m % GE::kMRows)
        hipLaunchKernelGGL((gemm_kernel<B, MODE, 0, GE, GS, ZPK>), dim3((unsigned)NT, 1, parts), block, 0, st, a,
                           one_rect(0, NT, F * GE::kMRows, 1, GE::kMRows));
}

// The layer GEMM for one group size and zero-point form (outl: accumulators seeded from the
// outlier partial, which the caller has computed).
template <int GS, int ZPK>
hipError_t gemm_main(int bits, bool outl, const GemmArgs &a, hipStream_t st)
{
    if (a.ksplit > 1) {  // k parts into fp32 partial rows (the caller sums them, outliers included)
        switch (bits) {
        case 2: gemm_launch<2, kSplitF32, GS, ZPK>(a, st); break;
        case 3: gemm_launch<3, kSplitF32, GS, ZPK>(a, st); break;
        case 4: gemm_launch<4, kSplitF32, GS, ZPK>(a, st); break;
        case 5: gemm_launch<5, kSplitF32, GS, ZPK>(a, st); break;
        case 6: gemm_launch<6, kSplitF32, GS, ZPK>(a, st); break;
        default: return hipErrorInvalidValue;
        }
    } else if constexpr (ZPK == kZpFp8) {  // fp8-scale weights carry no outliers
        if (outl) return hipErrorInvalidValue;
        switch (bits) {
        case 2: gemm_launch<2, kPlain, GS, ZPK>(a, st); break;
        case 3: gemm_launch<3, kPlain, GS, ZPK>(a, st); break;
        case 4: gemm_launch<4, kPlain, GS, ZPK>(a, st); break;
        case 5: gemm_launch<5, kPlain, GS, ZPK>(a, st); break;
        case 6: gemm_launch<6, kPlain, GS, ZPK>(a, st); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (bits) {
        case 2: outl ? gemm_launch<2, kOutl, GS, ZPK>(a, st) : gemm_launch<2, kPlain, GS, ZPK>(a, st); break;
        case 3: outl ? gemm_launch<3, kOutl, GS, ZPK>(a, st) : gemm_launch<3, kPlain, GS, ZPK>(a, st); break;
        case 4: outl ? gemm_launch<4, kOutl, GS, ZPK>(a, st) : gemm_launch<4, kPlain, GS, ZPK>(a, st); break;
        case 5: outl ? gemm_launch<5, kOutl, GS, ZPK>(a, st) : gemm_launch<5, kPlain, GS, ZPK>(a, st); break;
        case 6: outl ? gemm_launch<6, kOutl, GS, ZPK>(a, st) : gemm_launch<6, kPlain, GS, ZPK>(a, st); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

// Routed experts: one workgroup per (weight tile, occupied row tile of an expert's sorted
// rows).  The row counts live on the device, so the grid holds the most row tiles any routing
// of a.m rows over the experts can occupy, sum over e of ceil(c_e / T) <= (a.m + E (T - 1)) / T,
// and the surplus workgroups return at once.  With at most 32 rows per expert on average the
// small geometry runs (three 4-wave workgroups per CU instead of one 8-wave one), else the
// layer's.
template <int B, int MODE, typename GE, int GS, int ZPK>
hipError_t grouped_geo(int n_experts, const GemmArgs &a, hipStream_t st)
{
    constexpr int64_t T = GE::kMRows;
    const int64_t n_tiles = (a.n + GE::kNT - 1) / GE::kNT;
    const int64_t items = std::min<int64_t>((a.m + n_experts * (T - 1)) / T, n_experts * ((a.m + T - 1) / T));
    TilePlan plan{};
    plan.experts = n_experts;
    const unsigned parts = MODE == kGroupRowsF32 && a.ksplit > 1 ? (unsigned)a.ksplit : 1u;
    if (items > 65535) return hipErrorInvalidValue;  // refused by the caller's validation
    hipLaunchKernelGGL((gemm_kernel<B, MODE, 0, GE, GS, ZPK>), dim3((unsigned)n_tiles, (unsigned)items, parts),
                       dim3(GE::kWaves * 64), 0, st, a, plan);
    return hipGetLastError();
}
template <int B, int MODE, int GS, int ZPK>
hipError_t grouped_mode(int n_experts, const GemmArgs &a, hipStream_t st)
{
    if (a.m <= (int64_t)GeoExperts::kMRows * n_experts) return grouped_geo<B, MODE, GeoExperts, GS, ZPK>(n_experts, a, st);
    return grouped_geo<B, MODE, GeoLayer, GS, ZPK>(n_experts, a, st);
}
template <int B, int GS, int ZPK>
hipError_t grouped_bits(int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    switch (epilogue) {
    case QP_EPI_NONE: return grouped_mode<B, kGroupNone, GS, ZPK>(n_experts, a, st);
    case QP_EPI_SWIGLU: return grouped_mode<B, kGroupSwiglu, GS, ZPK>(n_experts, a, st);
    case QP_EPI_ROWS_F32: return grouped_mode<B, kGroupRowsF32, GS, ZPK>(n_experts, a, st);
    }
    return hipErrorInvalidValue;
}
template <int GS, int ZPK>
hipError_t grouped_main(int bits, int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    switch (bits) {
    case 2: return grouped_bits<2, GS, ZPK>(epilogue, n_experts, a, st);
    case 3: return grouped_bits<3, GS, ZPK>(epilogue, n_experts, a, st);
    case 4: return grouped_bits<4, GS, ZPK>(epilogue, n_experts, a, st);
    case 5: return grouped_bits<5, GS, ZPK>(epilogue, n_experts, a, st);
    case 6: return grouped_bits<6, GS, ZPK>(epilogue, n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

// Each variant is instantiated in one translation unit (they compile in parallel); the layer
// and grouped halves of a variant can also go to translation units of their own.
#define QP_GEMM_LAYER(GS, ZPK) template hipError_t gemm_main<GS, ZPK>(int, bool, const GemmArgs &, hipStream_t);
#define QP_GEMM_GROUPED(GS, ZPK) \
    template hipError_t grouped_main<GS, ZPK>(int, int, int, const GemmArgs &, hipStream_t);
#define QP_GEMM_VARIANT(GS, ZPK) QP_GEMM_LAYER(GS, ZPK) QP_GEMM_GROUPED(GS, ZPK)
#define QP_GEMM_VARIANT_EXTERN(GS, ZPK)                                                               \
    extern template hipError_t gemm_main<GS, ZPK>(int, bool, const GemmArgs &, hipStream_t);          \
    extern template hipError_t grouped_main<GS, ZPK>(int, int, int, const GemmArgs &, hipStream_t);

}  // namespace gk
}  // namespace qp
