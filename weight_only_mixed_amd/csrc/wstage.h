// Weight staging shared by the matrix-core GEMMs (fp16 and int8 activations).
//
// Both kernels read the device layout the same way: per k-loop step, each wave DMAs its two
// 16-row weight blocks of a k-tile from HBM into its own part of a two-slot LDS ring, loads the
// tile's scales and zero points into registers, and reads its lane chunk back from LDS to
// unpack it; the activation tile of each 128-k group is DMA'd into a two-slot LDS ring shared by
// the workgroup.  Waits are explicit (vmcnt counts and one barrier per step).
#pragma once

#include "bufio.h"

namespace qp {
namespace mm {

constexpr int kRBW = 2;             // 16-row weight blocks per wave

// LDS staging of one wave's row block for one k-tile: the lane chunks as in the device layout
// (B/2 pieces of 16 bytes per lane; for odd B the 8-byte tail as two 4-byte words 256 bytes
// apart).
template <int B>
struct WStage {
    static constexpr int kBytes = 512 * B;
    static constexpr int kOps = B / 2 + 2 * (B & 1);  // DMA instructions per row block
};
template <int B>
constexpr int kWOps = kRBW * WStage<B>::kOps;  // weight DMA instructions per wave per k-tile

// Buffers of one workgroup.  Every wave-uniform offset passed as soffset stays inside the
// range the per-lane voffset was checked against (a row of x, a weight row block), so a
// load is in bounds whether or not the hardware includes soffset in its range check.
constexpr int kDmaXMax = 4;  // activation DMA pieces per wave per group, at most
struct Bufs {
    rsrc_t x;                 // activation rows [m0, m)
    rsrc_t w[kRBW];           // packed tiles of row block rb0 + u (empty past the last block)
    rsrc_t sc[kRBW], zr[kRBW];
    uint32_t xoff[kDmaXMax];  // this lane's source of LDS-DMA piece it (row offset + chunk)
    uint32_t zmid;            // 0: stored zero points; else the implied pair used instead
};

__device__ __forceinline__ void lds_dma16(rsrc_t r, uint8_t *lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, uint8_t *lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, soff, 0, 0);
}

// DMA this wave's packed tiles of k-tile kt into its part `dst` of a weight slot.
template <int B>
__device__ __forceinline__ void dma_w(const Bufs &bf, int64_t kt, uint8_t *dst, int lane)
{
    const uint32_t tile = __builtin_amdgcn_readfirstlane((uint32_t)(kt * (512 * B)));
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        uint8_t *base = dst + u * WStage<B>::kBytes;
#pragma unroll
        for (int s = 0; s < B / 2; ++s) lds_dma16(bf.w[u], base + 1024 * s, 16 * lane, tile + 1024 * s);
        if constexpr (B & 1) {
            lds_dma4(bf.w[u], base + 1024 * (B / 2), 8 * lane, tile + 1024 * (B / 2));
            lds_dma4(bf.w[u], base + 1024 * (B / 2) + 256, 8 * lane + 4, tile + 1024 * (B / 2));
        }
    }
}

// This lane's chunk of one staged row block.
template <int B>
__device__ __forceinline__ void read_chunk(const uint8_t *base, int lane, uint32_t *d)
{
#pragma unroll
    for (int s = 0; s < B / 2; ++s) {
        const u4 v = *(const u4 *)(base + 1024 * s + 16 * lane);
        d[4 * s + 0] = v[0];
        d[4 * s + 1] = v[1];
        d[4 * s + 2] = v[2];
        d[4 * s + 3] = v[3];
    }
    if constexpr (B & 1) {
        d[2 * B - 2] = *(const uint32_t *)(base + 1024 * (B / 2) + 4 * lane);
        d[2 * B - 1] = *(const uint32_t *)(base + 1024 * (B / 2) + 256 + 4 * lane);
    }
}

// Scales and zero points of one k-tile (both groups) for this lane: the zero points of its
// weight row r, the scales of the accumulator rows 4t + i.
struct SZ {
    uint32_t zz[kRBW];
    uint32_t sc[kRBW][4];
};
constexpr int kSZOps = kRBW * 5;

__device__ __forceinline__ void load_sz(const Bufs &bf, int64_t G, int64_t kt, int lane, SZ &z)
{
    const int t = lane >> 4, r = lane & 15;
    const uint32_t vz = (uint32_t)(r * G), vs = (uint32_t)(4 * t * G * 2);
    const uint32_t zo = __builtin_amdgcn_readfirstlane((uint32_t)(2 * kt));
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        z.zz[u] = ld2(bf.zr[u], vz, zo);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            z.sc[u][i] = ld4(bf.sc[u], vs, __builtin_amdgcn_readfirstlane((uint32_t)((i * G + 2 * kt) * 2)));
    }
}

// The loads one k-loop step issues for later steps: the activation DMA of group gx into
// slot xdst, and on even steps (PAR 0) the scales and zero points of tile kt into z, on odd
// steps (PAR 1) the weight DMA of tile kt into this wave's part wdst of a weight slot.
template <int PAR>
struct StepIO {
    int64_t gx, kt;
    uint8_t *xdst, *wdst;
    SZ *z;
};

// Scale / zero-point load p of 2 x 5: the zero pair, then the four scale words of row block p / 5.
__device__ __forceinline__ void load_sz_piece(const Bufs &bf, int64_t G, int64_t kt, int lane, SZ &z, int p)
{
    const int t = lane >> 4, r = lane & 15, u = p / 5, j = p % 5;
    if (j == 0) {
        z.zz[u] = ld2(bf.zr[u], (uint32_t)(r * G), __builtin_amdgcn_readfirstlane((uint32_t)(2 * kt)));
    } else {
        const int i = j - 1;
        z.sc[u][i] = ld4(bf.sc[u], (uint32_t)(4 * t * G * 2), __builtin_amdgcn_readfirstlane((uint32_t)((i * G + 2 * kt) * 2)));
    }
}

// Weight DMA piece p of kWOps<B>: row block p / kOps, then its 16-byte pieces and (odd B) the
// two 4-byte words of the tail.
template <int B>
__device__ __forceinline__ void dma_w_piece(const Bufs &bf, int64_t kt, uint8_t *dst, int lane, int p)
{
    const uint32_t tile = __builtin_amdgcn_readfirstlane((uint32_t)(kt * (512 * B)));
    const int u = p / WStage<B>::kOps, s = p % WStage<B>::kOps;
    uint8_t *base = dst + u * WStage<B>::kBytes;
    if (s < B / 2) {
        lds_dma16(bf.w[u], base + 1024 * s, 16 * lane, tile + 1024 * s);
    } else {
        const int h = s - B / 2;  // tail word 0 or 1
        lds_dma4(bf.w[u], base + 1024 * (B / 2) + 256 * h, 8 * lane + 4 * h, tile + 1024 * (B / 2));
    }
}

// After a wait that has retired this tile's scale / zero-point loads: hide their origin from
// the compiler, which does not see the inline-asm wait and would otherwise wait for them again
// at their first use, counting the weight DMA issued since (meant to stay in flight) as older.
// Implied zero points (zmid != 0) replace the loaded ones (those loads read out of range).
__device__ __forceinline__ void retired(SZ &z, uint32_t zmid)
{
    if (zmid) {  // uniform
#pragma unroll
        for (int u = 0; u < kRBW; ++u) z.zz[u] = zmid;
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        asm volatile("" : "+v"(z.zz[u]));
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(z.sc[u][i]));
    }
}

// Wait until at most N of this wave's vector-memory operations are outstanding (they retire
// in order) and its LDS reads are done, then synchronise the workgroup.  The barrier is issued
// in the same asm statement: __syncthreads() carries a workgroup fence, for which the compiler
// waits for every outstanding buffer-to-LDS DMA (vmcnt(0)), including the ones issued this
// step to run ahead.  The DMA whose data the next step reads has landed once this wave's
// vmcnt allows it, so the plain barrier is enough; the memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_and_sync()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace mm
}  // namespace qp
