// Integer-dot dequant-GEMM: int8 activations x b-bit weights on the gfx950 int8 matrix cores.
//
// The inference acceleration guide (s1.2, s3.5) runs prefill with 8-bit activations so the
// products use the integer matrix units; the mixed-bit page (s4.2) gives the inner loop: unpack
// the b-bit codes to 8-bit integers, accumulate integer dot products, and apply the scale in
// fp32.  Per 128-k group g, for weight row n and activation row m:
//     isum = sum over k in g of xq[m][k] * (q[n][k] - zp[n][g])      (exact, int32)
//     acc[m][n] += s_w[n][g] * isum                                   (fp32)
// and y[m][n] = fp16(acc * s_x[m]) once at the end.
//
// The workgroup has the fp16 GEMM's structure: eight waves of two 16-row weight blocks (256
// rows), the same two-slot LDS rings filled by buffer-to-LDS DMA, the same weight staging, scale
// and zero-point loads and waits.  It covers 256 activation rows instead of 128: every output
// costs two vector ops per group here (conversion and fma) against one matrix-core op per 64 k,
// so the vector ALU sets the pace, and sixteen 16-row tiles per wave halve the unpack work per
// output (measured 17-25% faster than eight tiles at 2-6 bits; 241-250 VGPRs, no spills).
// What changes is the operand:
//  - Weights become the A operand of v_mfma_i32_16x16x64_i8 as bytes (q - zp).  A lane's
//    chunk holds, per 128-k group, four 8-k blocks (k = 32s + 8t + [0, 8) for lane quarter t);
//    blocks 2p and 2p+1 form its 16 bytes for matrix-core step p (p = 0, 1).  The codes are
//    moved to byte lanes with masks, shifts and byte permutes, the zero point is subtracted
//    four bytes at a time ((q + 128 - zp) has no borrow between bytes, XOR 0x80 makes it the
//    signed difference).
//  - Activations (the B operand) come from the int8 storage map of qpack.h, where one 16-byte
//    piece is exactly a lane's 16 k for one step; a 128-k group of one row is 128 bytes.  The
//    LDS slot keeps each row's eight pieces XOR-swizzled by row / 2, so a fragment read (16
//    rows, one piece each) covers 16 distinct 16-byte bank groups.
//  - Each group's integer result is converted and scaled right away (one conversion and one
//    fp32 fma per output), interleaved with the next group's unpack and the matrix-core chain
//    of the next activation tile.
// Rows of the last activation block past m read zeros and are not stored.  Outliers are not
// applied here (the held-out weights are fp16 and would need the fp16 activations).
#include <utility>

#include "unpack.h"
#include "wstage.h"

namespace qp {

namespace {

using namespace mm;

typedef int32_t i4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8, kMT = 16;
constexpr int kNT = kWaves * kRBW * kTileN;     // weight rows per workgroup
constexpr int kMRows = kMT * 16;                // activation rows per workgroup
constexpr int kXRow = 128;                      // bytes of one activation row per group
constexpr int kXSlot = kMRows * kXRow;          // one activation slot
constexpr int kDmaX = kXSlot / 1024 / kWaves;   // activation DMA pieces per wave per group
static_assert(kDmaX * 1024 * kWaves == kXSlot && kDmaX <= kDmaXMax, "whole 1 KB runs per wave");

template <int B>
struct Smem8 {
    uint8_t xs[2][kXSlot];
    uint8_t ws[2][kWaves * kRBW * WStage<B>::kBytes];
};

// LDS offset of piece c (0..7) of activation row `row` within a slot.
__device__ __forceinline__ int xs_off8(int row, int c) { return row * kXRow + ((c ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ i4v mfma8(i4v a, i4v b, i4v c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Activation DMA piece `it` of this wave for group g: run 2 wv + it of the slot, rows
// 8 run .. 8 run + 7; lane L writes LDS bytes [16 L, 16 L + 16) of the run = row 8 run + L / 8,
// physical piece L % 8, which holds logical piece (L % 8) ^ ((row >> 1) & 7).
__device__ __forceinline__ void dma_x8(const Bufs &bf, int64_t g, uint8_t *dst, int wv, int it)
{
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)g * kXRow);
    lds_dma16(bf.x, dst + (wv * kDmaX + it) * 1024, bf.xoff[it], soff);
}

// ---- unpack to int8 (q - zp) -------------------------------------------------------------

// Per-byte 0x80 - zp (zp < 64): added to bytes q < 64 it gives q + 128 - zp in [65, 191].
__device__ __forceinline__ uint32_t zbias(uint32_t zp) { return 0x80808080u - zp * 0x01010101u; }
__device__ __forceinline__ uint32_t to_s8(uint32_t w, uint32_t zb) { return (w + zb) ^ 0x80808080u; }

// Chunk bit of value v (0..7, k order) of block J, from the device layout's pair placement.
template <int B, int J, int V>
constexpr int val_pos()
{
    using R = PairRule<B, J, V / 2>;
    return V % 2 == 0 ? R::ABS + R::PLO : R::ABS + 16 + R::PHI;
}

// B-bit field at chunk bit P of d[2B].
template <int B, int P>
__device__ __forceinline__ uint32_t field(const uint32_t *d)
{
    constexpr int w = P / 32, o = P % 32;
    if constexpr (o + B <= 32)
        return __builtin_amdgcn_ubfe(d[w], o, B);
    else
        return __builtin_amdgcn_alignbit(d[w + 1], d[w], o) & ((1u << B) - 1);
}

// Four values V0..V0+3 of block J as bytes, k order.
template <int B, int J, int V0>
__device__ __forceinline__ uint32_t bytes4(const uint32_t *d)
{
    uint32_t w = field<B, val_pos<B, J, V0>()>(d);
    w |= field<B, val_pos<B, J, V0 + 1>()>(d) << 8;
    w |= field<B, val_pos<B, J, V0 + 2>()>(d) << 16;
    w |= field<B, val_pos<B, J, V0 + 3>()>(d) << 24;
    return w;
}

// Block J (0..7) of chunk d as eight signed bytes (q - zp) in k order: out[0] = k 0..3,
// out[1] = k 4..7.  4 bits: one word per block, v_{2i} at bit 4i and v_{2i+1} at 16 + 4i, so
// the low nibbles are (v0, v4, v1, v5), the high ones (v2, v6, v3, v7); two permutes order them.
template <int B, int J>
__device__ __forceinline__ void block_s8(const uint32_t *d, uint32_t zb, uint32_t *out)
{
    if constexpr (B == 4) {
        const uint32_t lo = d[J] & 0x0F0F0F0Fu, hi = (d[J] >> 4) & 0x0F0F0F0Fu;
        out[0] = to_s8(__builtin_amdgcn_perm(hi, lo, 0x06040200u), zb);
        out[1] = to_s8(__builtin_amdgcn_perm(hi, lo, 0x07050301u), zb);
    } else {
        out[0] = to_s8(bytes4<B, J, 0>(d), zb);
        out[1] = to_s8(bytes4<B, J, 4>(d), zb);
    }
}

// 2 bits: blocks 2j and 2j+1 share word d[j]; value 2i of block 2j + s sits at bit 8s + 2i, value
// 2i+1 at 16 + 8s + 2i.  f_i = (d >> 2i) & 0x03030303 holds (blk0 v_2i, blk1 v_2i, blk0 v_2i+1,
// blk1 v_2i+1); permutes of (f0, f1) and (f2, f3) give both blocks in k order.
template <int JP>
__device__ __forceinline__ void block_pair_s8_2(const uint32_t *d, uint32_t zb, uint32_t *out0, uint32_t *out1)
{
    const uint32_t w = d[JP];
    const uint32_t f0 = w & 0x03030303u, f1 = (w >> 2) & 0x03030303u;
    const uint32_t f2 = (w >> 4) & 0x03030303u, f3 = (w >> 6) & 0x03030303u;
    out0[0] = to_s8(__builtin_amdgcn_perm(f1, f0, 0x06040200u), zb);
    out0[1] = to_s8(__builtin_amdgcn_perm(f3, f2, 0x06040200u), zb);
    out1[0] = to_s8(__builtin_amdgcn_perm(f1, f0, 0x07050301u), zb);
    out1[1] = to_s8(__builtin_amdgcn_perm(f3, f2, 0x07050301u), zb);
}

// Operand words of block s (0..3) of group half NH: Wn[s / 2] words 2 (s % 2), 2 (s % 2) + 1.
template <int B, int NH, int S>
__device__ __forceinline__ void unpack_block8(const uint32_t *d, uint32_t zb, i4v (&Wn)[2])
{
    constexpr int J = 4 * NH + S;
    uint32_t o[2];
    block_s8<B, J>(d, zb, o);
    Wn[S / 2][2 * (S % 2)] = (int32_t)o[0];
    Wn[S / 2][2 * (S % 2) + 1] = (int32_t)o[1];
}
template <int NH, int S>
__device__ __forceinline__ void unpack_pair8_2(const uint32_t *d, uint32_t zb, i4v (&Wn)[2])
{
    constexpr int J = 4 * NH + S;  // S even: blocks J, J + 1 share word J / 2
    uint32_t o0[2], o1[2];
    block_pair_s8_2<J / 2>(d, zb, o0, o1);
    Wn[S / 2][0] = (int32_t)o0[0];
    Wn[S / 2][1] = (int32_t)o0[1];
    Wn[S / 2][2] = (int32_t)o1[0];
    Wn[S / 2][3] = (int32_t)o1[1];
}

// Unpack schedule over the activation tiles of a step: both row blocks' chunks are read at tile 0
// and unpacked from tile 1 on, when the reads have landed behind tile 0's matrix-core work.  The
// units (eight blocks, block / 4 = row block; 2 bits: four words of two blocks each) are spread
// evenly: unit j on tile 1 + j (kMT - 1) / units.
template <int B>
constexpr int kUnits = B == 2 ? 4 : 8;
template <int B>
constexpr int unit_tile(int j) { return 1 + j * (kMT - 1) / kUnits<B>; }

template <int B, int NH, int J>
__device__ __forceinline__ void unpack_unit(const uint32_t (&d)[kRBW][2 * B], const uint32_t (&zb)[kRBW],
                                            i4v (&Wn)[kRBW][2])
{
    constexpr int blk = B == 2 ? 2 * J : J, u = blk / 4, s = blk % 4;
    if constexpr (B == 2)
        unpack_pair8_2<NH, s>(d[u], zb[u], Wn[u]);
    else
        unpack_block8<B, NH, s>(d[u], zb[u], Wn[u]);
}
template <int B, int NH, int MT, int J>
__device__ __forceinline__ void unpack_if(const uint32_t (&d)[kRBW][2 * B], const uint32_t (&zb)[kRBW],
                                          i4v (&Wn)[kRBW][2])
{
    if constexpr (unit_tile<B>(J) == MT) unpack_unit<B, NH, J>(d, zb, Wn);
}
template <int B, int NH, int MT, int... J>
__device__ __forceinline__ void unpack_units(std::integer_sequence<int, J...>, const uint32_t (&d)[kRBW][2 * B],
                                             const uint32_t (&zb)[kRBW], i4v (&Wn)[kRBW][2])
{
    (unpack_if<B, NH, MT, J>(d, zb, Wn), ...);
}
template <int B, int NH, int MT>
__device__ __forceinline__ void unpack_share(const uint32_t (&d)[kRBW][2 * B], const uint32_t (&zb)[kRBW],
                                             i4v (&Wn)[kRBW][2])
{
    unpack_units<B, NH, MT>(std::make_integer_sequence<int, kUnits<B>>{}, d, zb, Wn);
}

template <int B, int NH, int... J>
__device__ __forceinline__ void unpack_all(std::integer_sequence<int, J...>, const uint32_t (&d)[kRBW][2 * B],
                                           const uint32_t (&zb)[kRBW], i4v (&Wn)[kRBW][2])
{
    (unpack_unit<B, NH, J>(d, zb, Wn), ...);
}

// Whole group (before the loop): both row blocks from a staged weight slot part.
template <int B, int NH>
__device__ __forceinline__ void unpack_group8(const uint8_t *wpart, const SZ<kGroup> &z, int lane, i4v (&W)[kRBW][2])
{
    uint32_t zb[kRBW];
#pragma unroll
    for (int u = 0; u < kRBW; ++u) zb[u] = zbias(zp_of(z, u, NH));
    uint32_t d[kRBW][2 * B];
    read_chunk<B>(wpart, lane, d[0]);
    read_chunk<B>(wpart + WStage<B>::kBytes, lane, d[1]);
    unpack_all<B, NH>(std::make_integer_sequence<int, kUnits<B>>{}, d, zb, W);
}

// ---- k loop --------------------------------------------------------------------------------

// tot[.][mt] += s * float(isum), s the scale of group SH of the tile for the lane's weight row.
template <int SH>
__device__ __forceinline__ void scale8(const SZ<kGroup> &zs, const i4v (&acc)[kRBW], f4 (&tot)[kRBW][kMT], int mt)
{
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const float s = sc_of(zs, u, SH);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[u][mt][i] = __builtin_fmaf(s, (float)acc[u][i], tot[u][mt][i]);
        asm volatile("" : "+v"(tot[u][mt]));
    }
}

// A step's loads for later steps, spread over its tiles: activation pieces with the first
// tiles; scales and zero points (even steps) with the first half; the weight DMA (odd steps)
// with the second half, after every activation piece, so the end-of-step wait can leave it in
// flight.
template <int B, int ZPK, int PAR, int MT>
__device__ __forceinline__ void issue_tile8(const Bufs &bf, const StepIO<PAR, kGroup> &io, int64_t G, int wv, int lane)
{
    if constexpr (MT < kDmaX) dma_x8(bf, io.gx, io.xdst, wv, MT);
    if constexpr (PAR == 0 && MT < kMT / 2) {
#pragma unroll
        for (int p = MT * kSZOps / (kMT / 2); p < (MT + 1) * kSZOps / (kMT / 2); ++p) load_sz_piece<B, kGroup, ZPK>(bf, G, io.kt, lane, *io.z, p);
    }
    if constexpr (PAR == 1 && MT >= kMT / 2) {
        constexpr int q = MT - kMT / 2, h = kMT / 2;
#pragma unroll
        for (int p = q * kWOps<B> / h; p < (q + 1) * kWOps<B> / h; ++p) dma_w_piece<B>(bf, io.kt, io.wdst, lane, p);
    }
}

constexpr int kXA = 1, kXR = kXA + 1;  // fragment reads run one tile ahead (ring of two)
constexpr int kLag = 1, kAR = kLag + 1;  // integer sums are scaled one tile later (ring of two)

// Activation tile MT of a step: its fragment reads for tile MT + 2, the matrix-core chains of
// tile MT (two K = 64 steps per row block, from zero), the scaling of tile MT - 2's integer
// sums (their matrix-core ops finished a tile ago) and a share of the next group's unpack.
template <int B, int ZPK, int SH, int NH, int MT>
__device__ __forceinline__ void tile8(const i4v (&Wc)[kRBW][2], i4v (&Wn)[kRBW][2], const SZ<kGroup> &zs,
                                      const uint32_t (&zb)[kRBW], const uint8_t *xs, const uint8_t *wpart, int lane,
                                      uint32_t (&d)[kRBW][2 * B], i4v (&X)[kXR][2], i4v (&acc)[kAR][kRBW],
                                      f4 (&tot)[kRBW][kMT], const Bufs &bf, const StepIO<NH ^ 1, kGroup> &io, int64_t G, int wv)
{
    constexpr int cur = MT % kAR;
    const int t = lane >> 4, r = lane & 15;
    issue_tile8<B, ZPK, NH ^ 1, MT>(bf, io, G, wv, lane);
    if constexpr (MT + kXA < kMT) {
#pragma unroll
        for (int p = 0; p < 2; ++p) X[(MT + kXA) % kXR][p] = *(const i4v *)(xs + xs_off8(16 * (MT + kXA) + r, 4 * p + t));
    }
    if constexpr (MT == 0) read_chunk<B>(wpart, lane, d[0]);
    if constexpr (MT == 0) read_chunk<B>(wpart + WStage<B>::kBytes, lane, d[1]);
#pragma unroll
    for (int u = 0; u < kRBW; ++u) acc[cur][u] = mfma8(X[MT % kXR][0], Wc[u][0], (i4v){0, 0, 0, 0});
#pragma unroll
    for (int u = 0; u < kRBW; ++u) acc[cur][u] = mfma8(X[MT % kXR][1], Wc[u][1], acc[cur][u]);
    unpack_share<B, NH, MT>(d, zb, Wn);
    if constexpr (MT >= kLag) scale8<SH>(zs, acc[(MT - kLag) % kAR], tot, MT - kLag);
    if constexpr (MT == kMT - 1) {
#pragma unroll
        for (int j = kMT - kLag; j < kMT; ++j) scale8<SH>(zs, acc[j % kAR], tot, j);
    }
    // per matrix-core op: a fragment read and a few vector ops issued behind it
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int B, int ZPK, int SH, int NH, int... MT>
__device__ __forceinline__ void tiles8(std::integer_sequence<int, MT...>, const i4v (&Wc)[kRBW][2], i4v (&Wn)[kRBW][2],
                                       const SZ<kGroup> &zs, const uint32_t (&zb)[kRBW], const uint8_t *xs,
                                       const uint8_t *wpart, int lane, uint32_t (&d)[kRBW][2 * B], i4v (&X)[kXR][2],
                                       i4v (&acc)[kAR][kRBW], f4 (&tot)[kRBW][kMT], const Bufs &bf,
                                       const StepIO<NH ^ 1, kGroup> &io, int64_t G, int wv)
{
    (tile8<B, ZPK, SH, NH, MT>(Wc, Wn, zs, zb, xs, wpart, lane, d, X, acc, tot, bf, io, G, wv), ...);
}

// One 128-k group step: Wc times the activation tile of this group (slot xs), scale half SH;
// meanwhile the next group (half NH of staged tile wpart, zero points zn) is unpacked into Wn
// and the loads io are issued.
template <int B, int ZPK, int SH, int NH>
__device__ __forceinline__ void step8(const i4v (&Wc)[kRBW][2], i4v (&Wn)[kRBW][2], const SZ<kGroup> &zs,
                                      const SZ<kGroup> &zn, const uint8_t *xs, const uint8_t *wpart, int lane,
                                      f4 (&tot)[kRBW][kMT], const Bufs &bf, const StepIO<NH ^ 1, kGroup> &io, int64_t G, int wv)
{
    const int t = lane >> 4, r = lane & 15;
    i4v X[kXR][2];
#pragma unroll
    for (int mt = 0; mt < kXA; ++mt)
#pragma unroll
        for (int p = 0; p < 2; ++p) X[mt][p] = *(const i4v *)(xs + xs_off8(16 * mt + r, 4 * p + t));
    uint32_t zb[kRBW];
#pragma unroll
    for (int u = 0; u < kRBW; ++u) zb[u] = zbias(zp_of(zn, u, NH));
    uint32_t d[kRBW][2 * B];
    i4v acc[kAR][kRBW];
    __builtin_amdgcn_sched_barrier(0);
    tiles8<B, ZPK, SH, NH>(std::make_integer_sequence<int, kMT>{}, Wc, Wn, zs, zb, xs, wpart, lane, d, X, acc, tot, bf, io,
                      G, wv);
}

// The k loop: the fp16 GEMM's schedule.  Step g multiplies group g (activation slot g % 2) and
// unpacks group g + 1; weight slot t % 2 holds k-tile t, read in steps 2t - 1 and 2t and
// refilled with tile t + 2 during step 2t + 1; scales and zero points of tile t are loaded
// during step 2t - 2.  Waits: vmcnt(0) after even steps, vmcnt(weight DMAs) after odd ones.
// Loads past the end are clamped to the last group or tile; what is unpacked from them is
// discarded.
template <int B, int ZPK>
__device__ __forceinline__ void k_loop8(const Bufs &bf, uint8_t *__restrict__ xs0, uint8_t *__restrict__ xs1,
                                        uint8_t *__restrict__ ws0, uint8_t *__restrict__ ws1, int64_t KT, int64_t G,
                                        int wv, int lane, f4 (&tot)[kRBW][kMT])
{
    const int64_t GN = 2 * KT;
    auto gclamp = [&](int64_t g) { return g < GN ? g : GN - 1; };
    auto tclamp = [&](int64_t t) { return t < KT ? t : KT - 1; };
    uint8_t *w0 = ws0 + wv * (kRBW * WStage<B>::kBytes);
    uint8_t *w1 = ws1 + wv * (kRBW * WStage<B>::kBytes);
    SZ<kGroup> z0{}, z1{};
    i4v Wa[kRBW][2], Wb[kRBW][2];

#pragma unroll
    for (int it = 0; it < kDmaX; ++it) dma_x8(bf, 0, xs0, wv, it);
    dma_w<B>(bf, 0, w0, lane);
    dma_w<B>(bf, tclamp(1), w1, lane);
    load_sz<B, kGroup, ZPK>(bf, G, 0, lane, z0);
    wait_and_sync<0>();
    retired<B, kGroup, ZPK>(z0, bf, 0);
    unpack_group8<B, 0>(w0, z0, lane, Wa);

    for (int64_t kt = 0; kt < KT; kt += 2) {
        const int64_t g = 2 * kt;
        const StepIO<0, kGroup> s0{gclamp(g + 1), tclamp(kt + 1), xs1, nullptr, &z1};
        step8<B, ZPK, 0, 1>(Wa, Wb, z0, z0, xs0, w0, lane, tot, bf, s0, G, wv);
        wait_and_sync<0>();
        retired<B, kGroup, ZPK>(z1, bf, tclamp(kt + 1));
        const StepIO<1, kGroup> s1{gclamp(g + 2), tclamp(kt + 2), xs0, w0, nullptr};
        step8<B, ZPK, 1, 0>(Wb, Wa, z0, z1, xs1, w1, lane, tot, bf, s1, G, wv);
        wait_and_sync<kWOps<B>>();
        if (kt + 1 >= KT) break;
        const StepIO<0, kGroup> s2{gclamp(g + 3), tclamp(kt + 2), xs1, nullptr, &z0};
        step8<B, ZPK, 0, 1>(Wa, Wb, z1, z1, xs0, w1, lane, tot, bf, s2, G, wv);
        wait_and_sync<0>();
        retired<B, kGroup, ZPK>(z0, bf, tclamp(kt + 2));
        const StepIO<1, kGroup> s3{gclamp(g + 4), tclamp(kt + 3), xs0, w1, nullptr};
        step8<B, ZPK, 1, 0>(Wb, Wa, z1, z0, xs1, w0, lane, tot, bf, s3, G, wv);
        wait_and_sync<kWOps<B>>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may land after the workgroup ends
}

// Workgroup b -> (weight tile, activation block).  With a multiple of 8 weight tiles, the
// activation blocks of one weight tile get equal b % 8 (the same XCD, sharing its L2 copy of
// the packed weights).
__device__ __forceinline__ void plan8(int64_t b, int64_t NT, int64_t MB, int64_t &nt, int64_t &mb)
{
    if (NT % 8 == 0) {
        const int64_t xcd = b % 8, l8 = b / 8;
        nt = (l8 / MB) * 8 + xcd;
        mb = l8 % MB;
    } else {
        nt = b % NT;
        mb = b / NT;
    }
}

template <int B, int ZPK>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_a8_kernel(
    ExpertPtrs W, const int8_t *xq, const float *sx, int64_t m, int64_t n, int64_t k, uint32_t zmid, uint32_t zrow,
    uint16_t *y, int64_t ldy)
{
    __shared__ __attribute__((aligned(16))) Smem8<B> sm;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = k / kTileK, G = k / kGroup;
    const int64_t NT = (n + kNT - 1) / kNT, MB = (m + kMRows - 1) / kMRows;
    int64_t nt, mb;
    plan8(blockIdx.x, NT, MB, nt, mb);
    const int64_t m0 = mb * kMRows, NB = n / kTileN;
    const int64_t rb0 = nt * (kNT / kTileN) + wv * kRBW;

    Bufs bf;
    bf.zmid = zmid;
    bf.zrow = zrow;
    bf.kt0 = 0;
    bf.x = make_rsrc(xq, m * k);
    bf.rowf = make_rsrc(W.rowf, W.rowf ? n * 4 : 0);
    bf.row0 = (uint32_t)(rb0 * kTileN);
    bf.fb = make_rsrc(W.fb, W.fb ? n * W.fb_stride * 2 : 0);
    bf.fbs = W.fb_stride;
#pragma unroll
    for (int it = 0; it < kDmaX; ++it) {
        const int row = 8 * (kDmaX * wv + it) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        const int64_t sr = m0 + row;
        bf.xoff[it] = sr < m ? (uint32_t)(sr * k + 16 * c) : 0x80000000u;
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        const int64_t rb = rb0 + u;
        const bool in = rb < NB;
        bf.w[u] = make_rsrc(W.packed + rb * KT * (512 * B), in ? KT * (512 * B) : 0);
        if constexpr (ZPK == kZpFp8)  // scale bytes
            bf.sc[u] = make_rsrc((const uint8_t *)W.scales + rb * kTileN * G, in ? kTileN * G : 0);
        else
            bf.sc[u] = make_rsrc(W.scales + rb * kTileN * G, in ? kTileN * G * 2 : 0);
        const int64_t zstride = zrow ? zrow : G;  // zero-point bytes per weight row
        bf.zr[u] = make_rsrc(W.zeros + rb * kTileN * zstride, in && !zmid ? kTileN * zstride : 0);
    }

    f4 tot[kRBW][kMT];
#pragma unroll
    for (int u = 0; u < kRBW; ++u)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            tot[u][mt] = (f4){0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+v"(tot[u][mt]));
        }

    k_loop8<B, ZPK>(bf, sm.xs[0], sm.xs[1], sm.ws[0], sm.ws[1], KT, G, wv, lane, tot);

    // lane (t, r): activation rows 16 mt + 4 t + i of weight row rb * 16 + r
    float rowf[kRBW];  // fp8 scales: each row block's weight-row factor (1 otherwise)
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        rowf[u] = 1.0f;
        if constexpr (ZPK == kZpFp8)
            if (rb0 + u < NB) rowf[u] = W.rowf[(rb0 + u) * kTileN + r];
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = m0 + 16 * mt + 4 * t + i;
            if (row >= m) continue;
            const float s = sx[row];
#pragma unroll
            for (int u = 0; u < kRBW; ++u) {
                const int64_t rb = rb0 + u;
                if (rb >= NB) continue;
                float v = tot[u][mt][i];
                if constexpr (ZPK == kZpFp8) v *= rowf[u];
                y[row * ldy + rb * kTileN + r] = __builtin_bit_cast(uint16_t, (_Float16)(v * s));
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_a8(int bits, const ExpertPtrs &w, bool fp8, const int8_t *xq, const float *sx, int64_t m,
                          int64_t n, int64_t k, uint32_t zmid, uint32_t zrow, uint16_t *y, int64_t ldy, hipStream_t st)
{
    if (m < 1) return hipSuccess;
    const int64_t blocks = ((n + kNT - 1) / kNT) * ((m + kMRows - 1) / kMRows);
    const dim3 grid((unsigned)blocks), block(kWaves * 64);
    const int zpk = fp8 ? kZpFp8 : zrow ? kZpPacked : kZpByte;
    switch (bits * 3 + zpk) {
#define QP_A8_CASE(B, ZPK)                                                                                      \
    case B * 3 + ZPK:                                                                                           \
        hipLaunchKernelGGL((gemm_a8_kernel<B, ZPK>), grid, block, 0, st, w, xq, sx, m, n, k, zmid, zrow, y, ldy); \
        break;
        QP_A8_CASE(2, kZpByte) QP_A8_CASE(2, kZpPacked) QP_A8_CASE(2, kZpFp8)
        QP_A8_CASE(3, kZpByte) QP_A8_CASE(3, kZpPacked) QP_A8_CASE(3, kZpFp8)
        QP_A8_CASE(4, kZpByte) QP_A8_CASE(4, kZpPacked) QP_A8_CASE(4, kZpFp8)
        QP_A8_CASE(5, kZpByte) QP_A8_CASE(5, kZpPacked) QP_A8_CASE(5, kZpFp8)
        QP_A8_CASE(6, kZpByte) QP_A8_CASE(6, kZpPacked) QP_A8_CASE(6, kZpFp8)
#undef QP_A8_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qp
