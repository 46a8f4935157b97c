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
    uint32_t zmid;            // 0: stored zero points; else the implied zero point (low byte) used instead
    uint32_t zrow;            // b-bit zero points: bytes per row
    uint32_t kt0;             // first k-tile of this workgroup's k range (metadata is indexed from k = 0)
    // fp8 scales (ZPK == kZpFp8): row factors [n] and fp16 fallback lists [n][fbs] (buffer
    // ranges), the wave's first weight row
    rsrc_t rowf, fb;
    int32_t fbs;              // fallback slots per row
    uint32_t row0;
};

// Metadata forms (template parameter ZPK): fp16 scales with byte (or implied) zero points,
// fp16 scales with b-bit zero points, E4M3 scale bytes (times a row factor, fp16 fallback
// list) with byte (or implied) zero points.
enum { kZpByte = 0, kZpPacked = 1, kZpFp8 = 2 };

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

// Scales and zero points of one k-tile for this lane's weight rows: row r (lane % 16) of each
// of its two row blocks.  The tile holds kNGT = 256 / GS groups; group q's fp16 scale is half
// q % 2 of sc[u][q / 2], its zero point byte q % 4 of zz[u][q / 4].  b-bit zero points arrive as
// the two words of the row's bit stream that hold the tile's fields and are expanded to bytes
// by retired().
template <int GS>
struct SZ {
    static constexpr int kNGT = kTileK / GS, kSW = kNGT / 2;
    static_assert(GS == 32 || GS == 64 || GS == 128, "group size");
    uint32_t zz[kRBW][2];
    uint32_t sc[kRBW][kSW];    // as loaded: fp16 pairs
    float scf[kRBW][kNGT];     // converted once per tile by retired()
};
constexpr int kSZPer = 3;                // loads per row block: zero word 0, zero word 1, scales
constexpr int kSZOps = kRBW * kSZPer;    // scale / zero-point loads per wave per k-tile

// First bit of k-tile kt's fields in a row of b-bit zero points, and whether they run into a
// second 32-bit word.
template <int B, int GS>
__device__ __forceinline__ uint32_t zbit(int64_t kt) { return (uint32_t)(kt * SZ<GS>::kNGT * B); }
template <int B, int GS>
__device__ __forceinline__ bool zstraddles(int64_t kt) { return (zbit<B, GS>(kt) & 31) + SZ<GS>::kNGT * B > 32; }

// Load p of kSZOps: row block p / 3, then its zero word 0, zero word 1 (the next four byte
// zero points for g = 32; the second word of b-bit zero points that straddle one), the scales
// (4, 8 or 16 bytes).  Each load writes one fixed word, so the metadata stays in registers.
template <int B, int GS, int ZPK>
__device__ __forceinline__ void load_sz_piece(const Bufs &bf, int64_t G, int64_t ktl, int lane, SZ<GS> &z, int p)
{
    const int r = lane & 15, u = p / kSZPer, j = p % kSZPer;
    const int64_t kt = ktl + bf.kt0;
    if (j == 0) {
        if constexpr (ZPK == kZpPacked)
            z.zz[u][0] = ld4(bf.zr[u], (uint32_t)r * bf.zrow, uni(4 * (zbit<B, GS>(kt) >> 5)));
        else if constexpr (GS == 32)
            z.zz[u][0] = ld4(bf.zr[u], (uint32_t)(r * G), uni(8 * kt));
        else if constexpr (GS == 64)
            z.zz[u][0] = ld4(bf.zr[u], (uint32_t)(r * G), uni(4 * kt));
        else
            z.zz[u][0] = ld2(bf.zr[u], (uint32_t)(r * G), uni(2 * kt));
    } else if (j == 1) {
        if constexpr (ZPK == kZpPacked) {
            // the second word lies inside the row whenever the fields reach it
            if (zstraddles<B, GS>(kt)) z.zz[u][1] = ld4(bf.zr[u], (uint32_t)r * bf.zrow, uni(4 * (zbit<B, GS>(kt) >> 5) + 4));
        } else if constexpr (GS == 32) {
            z.zz[u][1] = ld4(bf.zr[u], (uint32_t)(r * G), uni(8 * kt + 4));
        }
    } else if constexpr (ZPK == kZpFp8) {  // one scale byte per group
        if constexpr (GS == 32) {
            const u2 v = ld8(bf.sc[u], (uint32_t)(r * G), uni(8 * kt));
            z.sc[u][0] = v[0];
            z.sc[u][1] = v[1];
        } else if constexpr (GS == 64) {
            z.sc[u][0] = ld4(bf.sc[u], (uint32_t)(r * G), uni(4 * kt));
        } else {
            z.sc[u][0] = ld2(bf.sc[u], (uint32_t)(r * G), uni(2 * kt));
        }
    } else {
        if constexpr (GS == 32) {
            const u4 v = ld16(bf.sc[u], (uint32_t)(r * G * 2), uni(16 * kt));
            z.sc[u][0] = v[0];
            z.sc[u][1] = v[1];
            z.sc[u][2] = v[2];
            z.sc[u][3] = v[3];
        } else if constexpr (GS == 64) {
            const u2 v = ld8(bf.sc[u], (uint32_t)(r * G * 2), uni(8 * kt));
            z.sc[u][0] = v[0];
            z.sc[u][1] = v[1];
        } else {
            z.sc[u][0] = ld4(bf.sc[u], (uint32_t)(r * G * 2), uni(4 * kt));
        }
    }
}

template <int B, int GS, int ZPK>
__device__ __forceinline__ void load_sz(const Bufs &bf, int64_t G, int64_t kt, int lane, SZ<GS> &z)
{
#pragma unroll
    for (int p = 0; p < kSZOps; ++p) load_sz_piece<B, GS, ZPK>(bf, G, kt, lane, z, p);
}

// Zero point and fp16 scale (as fp32) of group q (0 .. kNGT-1) of the tile, row block u.
template <int GS>
__device__ __forceinline__ uint32_t zp_of(const SZ<GS> &z, int u, int q)
{
    return (z.zz[u][q >> 2] >> (8 * (q & 3))) & 0xFF;
}
template <int GS>
__device__ __forceinline__ float sc_of(const SZ<GS> &z, int u, int q)
{
    return z.scf[u][q];
}

// The loads one k-loop step issues for later steps: the activation DMA of group gx into
// slot xdst, and on even steps (PAR 0) the scales and zero points of tile kt into z, on odd
// steps (PAR 1) the weight DMA of tile kt into this wave's part wdst of a weight slot.
template <int PAR, int GS>
struct StepIO {
    int64_t gx, kt;
    uint8_t *xdst, *wdst;
    SZ<GS> *z;
};

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

// After the wait that has retired the loads of k-tile kt's metadata: b-bit zero points (ZPK)
// are expanded to one byte per group; otherwise the implied zero point is added, replicated to
// every byte (0 for stored zero points; the loads of implied ones read out of range, as zeros).
// The scales are converted to fp32 once, and the registers' origin is hidden from the
// compiler, which does not see the inline-asm wait and would otherwise wait for the loads
// again at their first use, counting the weight DMA issued since (meant to stay in flight) as
// older.  Branch-free: a branch here splits the k loop into blocks the scheduler cannot
// interleave across.
template <int B, int GS, int ZPK>
__device__ __forceinline__ void retired(SZ<GS> &z, const Bufs &bf, int64_t ktl)
{
    if constexpr (ZPK == kZpPacked) {
        const int64_t kt = ktl + bf.kt0;
        const uint32_t sh = zbit<B, GS>(kt) & 31;
        const bool two = zstraddles<B, GS>(kt);
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
            const uint64_t v = ((uint64_t)(two ? z.zz[u][1] : 0u) << 32 | z.zz[u][0]) >> sh;
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int q = 0; q < SZ<GS>::kNGT; ++q) w[q >> 2] |= (uint32_t)((v >> (q * B)) & ((1u << B) - 1)) << (8 * (q & 3));
            z.zz[u][0] = w[0];
            z.zz[u][1] = w[1];
        }
    } else {
        const uint32_t rep = (bf.zmid & 0xFF) * 0x01010101u;
#pragma unroll
        for (int u = 0; u < kRBW; ++u) {
            z.zz[u][0] += rep;
            z.zz[u][1] += rep;
        }
    }
#pragma unroll
    for (int u = 0; u < kRBW; ++u) {
        asm volatile("" : "+v"(z.zz[u][0]), "+v"(z.zz[u][1]));
        // scale words holding data: fp16 pairs, or four E4M3 bytes per word
        constexpr int kWords = ZPK == kZpFp8 ? (SZ<GS>::kNGT + 3) / 4 : SZ<GS>::kSW;
#pragma unroll
        for (int i = 0; i < kWords; ++i) asm volatile("" : "+v"(z.sc[u][i]));
        // one conversion per group and tile (each scale multiplies four outputs per tile)
        if constexpr (ZPK == kZpFp8) {
            // two E4M3 bytes per conversion (the row factor multiplies the row's sums once, in
            // the epilogue); a byte with bit 7 set (rare) takes the fp16 scale from the row's
            // fallback list over the row factor instead, its index clamped to the list
            uint32_t esc = 0;
#pragma unroll
            for (int q = 0; q < SZ<GS>::kNGT; q += 2) {
                const uint32_t w = z.sc[u][q >> 2];
                const auto v = (q & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                                       : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
                z.scf[u][q] = v[0];
                z.scf[u][q + 1] = v[1];
                esc |= w;
            }
            if (esc & 0x80808080u) {
                const uint32_t row = bf.row0 + u * kTileN + (threadIdx.x & 15);
#pragma unroll
                for (int q = 0; q < SZ<GS>::kNGT; ++q) {
                    const uint32_t b = (z.sc[u][q >> 2] >> (8 * (q & 3))) & 0xFF;
                    if (b & 0x80) {
                        const int j = min((int)(b & 0x7F), bf.fbs - 1);
                        z.scf[u][q] = j >= 0 ? h_f(ld2(bf.fb, 2 * (row * (uint32_t)bf.fbs + (uint32_t)j))) *
                                                   __builtin_amdgcn_rcpf(as_f(ld4(bf.rowf, 4 * row)))
                                             : 0.0f;
                    }
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < SZ<GS>::kNGT; ++q) z.scf[u][q] = (q & 1) ? hi_h(z.sc[u][q >> 1]) : lo_h(z.sc[u][q >> 1]);
        }
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
