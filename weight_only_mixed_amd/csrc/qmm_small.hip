// Decode dequant-GEMV (m <= 16) on gfx950 matrix cores.
//
// The fused dequant-GEMM of the single-GPU 70B page (s3) is re-designed for CDNA4: packed
// weights stream from HBM in the device tile order, every lane unpacks its own eight 8-k blocks (the page units, mixed-bit page s3.2)
// into exact fp16 (q - zp) values, and one v_mfma_f32_16x16x32_f16 per block multiplies 16
// weight rows by up to 16 activation rows.  Activation rows beyond m are zero, so the matrix
// core reduces over k for every m <= 16 at the same cost; no cross-lane shuffle reduction is
// needed inside a wave.  Each 128-k group is accumulated separately in fp32 and scaled by its
// fp16 scale in fp32 (mixed-bit page, s4.2).  The outlier CSR is added in fp32 before the one
// fp16 rounding of y (70B page, s2).
//
// Scale and zero-point storage is a template mode (ZP): kMetaByte -- fp16 scales with byte
// (or implied) zero points; kMetaPacked -- fp16 scales with b-bit zero points; kMetaFp8 --
// E4M3 scale bytes times a per-row fp32 factor, with an fp16 fallback list (mixed-bit page,
// s2.3), and byte (or implied) zero points.  fp8 groups are accumulated with their E4M3 value
// and the row sum is multiplied by the row factor once, after the k reduction.
//
// Matrix-core fragment layout (A = 16 weight rows x 32 k, B = 32 k x 16 activation rows):
// lane l = 16*t + r supplies row r of A and column r of B for k-slots 8t..8t+7 and receives
// D[4t + i][r], i = 0..3 (weight row 4t+i, activation row r).
#include "bufio.h"
#include "unpack.h"

namespace qp {

enum { kMetaByte = 0, kMetaPacked = 1, kMetaFp8 = 2 };

// tot += sum over the tile's NG groups c of s_c * (A[j] . X[j] for the 8/NG blocks j of c),
// groups kept apart and added in group order.  sc[i][c / 2] holds the fp16 scales of groups
// c and c+1 (low, high half) for accumulator row 4t + i.
template <int NG>
__device__ __forceinline__ void mma_tile(const h8 *A, const h8 *X, const uint32_t (&sc)[4][NG / 2], f4 &tot)
{
    constexpr int JB = 8 / NG;  // blocks per group
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 acc[NG];
#pragma unroll
    for (int c = 0; c < NG; ++c) acc[c] = mfma16(A[c * JB], X[c * JB], z);
#pragma unroll
    for (int jj = 1; jj < JB; ++jj)
#pragma unroll
        for (int c = 0; c < NG; ++c) acc[c] = mfma16(A[c * JB + jj], X[c * JB + jj], acc[c]);
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            tot[i] = __builtin_fmaf((c & 1) ? hi_h(sc[i][c / 2]) : lo_h(sc[i][c / 2]), acc[c][i], tot[i]);
}

// As mma_tile, with the groups' scales as fp32 values: scf[i][c] for row 4t + i, group c.
template <int NG>
__device__ __forceinline__ void mma_tile_f(const h8 *A, const h8 *X, const float (&scf)[4][NG], f4 &tot)
{
    constexpr int JB = 8 / NG;
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 acc[NG];
#pragma unroll
    for (int c = 0; c < NG; ++c) acc[c] = mfma16(A[c * JB], X[c * JB], z);
#pragma unroll
    for (int jj = 1; jj < JB; ++jj)
#pragma unroll
        for (int c = 0; c < NG; ++c) acc[c] = mfma16(A[c * JB + jj], X[c * JB + jj], acc[c]);
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = __builtin_fmaf(scf[i][c], acc[c][i], tot[i]);
}

// Two E4M3 bytes (the low or high half of w) as fp32.
template <bool HI>
__device__ __forceinline__ void e4m3_pair(uint32_t w, float &a, float &b)
{
    const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    a = v[0];
    b = v[1];
}

// ---- decode GEMV: one workgroup per 16-row block, NW waves take its k-tiles round-robin --
//
// Decode is bound by the launch and the latency of each wave's few tiles at these sizes (a
// 4096 x 4096 layer is a few MB), not by bandwidth or vector work.  Every
// operand of a k-tile -- packed codes, the activation rows, scales and zero points -- is
// copied HBM -> LDS by buffer-to-LDS DMA into a per-wave ring of D slots, issued D-1 tiles
// ahead, so bytes in flight cost no registers and a CU holds many waves.  Each DMA reads at
// an offset checked by its buffer range: activation rows at or beyond m read as zeros, and
// tiles past the end of k read zeros into a slot that is never consumed, so every tile issues
// the same number of loads and one s_waitcnt count covers the ring.  A wave then unpacks the
// tile from LDS and multiplies it on the matrix core; lanes of activation rows >= m keep zero
// fragments and skip their LDS reads.  The NW partial sums of a row block are reduced
// through LDS in a fixed order, and the outlier CSR is added in fp32 before the fp16 store.

struct GemvBufs {
    rsrc_t w, sc, zr, x;
    uint32_t zrow;  // bytes per row of b-bit zero points (kMetaPacked); 0 otherwise
    int64_t G;
};

// One ring slot: a k-tile's packed codes, activation rows, and the scales and zero points of
// its NG = 256 / GS groups for the block's 16 rows (lane l < 16 stages row l; lanes >= 16 read
// zeros).  Scales: NG = 2 one 4-byte DMA, NG = 4 two (region A groups 0-1, B groups 2-3),
// NG = 8 one 16-byte DMA.  Zero points: NG = 2 the aligned 4-byte word holding the pair,
// NG = 4 one 4-byte DMA, NG = 8 two (groups 0-3, 4-7); b-bit zero points (ZP) the 32-bit
// words of the row's bit stream that cover the tile's NG fields (two, or three when
// NG*B + 31 > 64).  fp8 scale bytes are staged as byte zero points are.
template <int B, int MX, int GS, int ZP = kMetaByte>
struct RingSlot {
    static constexpr int NG = kTileK / GS;
    static constexpr int kScOps = ZP == kMetaFp8 ? (NG == 8 ? 2 : 1) : (NG == 4 ? 2 : 1);
    static constexpr int kZrOps = ZP == kMetaPacked ? (NG * B + 62) / 32 : (NG == 8 ? 2 : 1);
    static constexpr int kCodes = 512 * B;           // packed tile
    static constexpr int kX = kCodes;                 // activation rows, 512 B each, 2 per DMA
    static constexpr int kSc = kX + 1024 * MX;
    static constexpr int kZr = kSc + (NG == 8 && ZP != kMetaFp8 ? 1024 : 256 * kScOps);
    static constexpr int kBytes = kZr + 256 * kZrOps;
    static constexpr int kLoads = B / 2 + 2 * (B & 1) + MX + kScOps + kZrOps;  // DMA instructions per tile
    static_assert(NG == 2 || NG == 4 || NG == 8, "groups of 128, 64 or 32");
};

__device__ __forceinline__ void dma16(rsrc_t r, uint8_t *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint8_t *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

template <int B, int MX, int GS, int ZP>
__device__ __forceinline__ void ring_issue(const GemvBufs &bf, int64_t kt, int lane, int64_t ldx, uint8_t *slot)
{
    using S = RingSlot<B, MX, GS, ZP>;
    constexpr int NG = S::NG;
    const uint32_t tw = (uint32_t)(kt * (512 * B));
#pragma unroll
    for (int sl = 0; sl < B / 2; ++sl) dma16(bf.w, slot + 1024 * sl, tw + 1024 * sl + 16 * lane);
    if (B & 1) {
        dma4(bf.w, slot + 1024 * (B / 2), tw + 1024 * (B / 2) + 8 * lane);
        dma4(bf.w, slot + 1024 * (B / 2) + 256, tw + 1024 * (B / 2) + 8 * lane + 4);
    }
    const uint32_t xk = (uint32_t)(kt * (kTileK * 2));
#pragma unroll
    for (int q = 0; q < MX; ++q) {
        const uint32_t row = 2 * q + (lane >> 5);
        dma16(bf.x, slot + S::kX + 1024 * q, (uint32_t)(row * ldx * 2) + xk + 16 * (lane & 31));
    }
    const uint32_t g0 = (uint32_t)(lane * bf.G + NG * kt);  // this lane's row, the tile's first group
    if constexpr (ZP == kMetaFp8) {  // scale bytes, then zero points, each as byte zero points
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const rsrc_t &rs = e == 0 ? bf.sc : bf.zr;
            uint8_t *dst = slot + (e == 0 ? S::kSc : S::kZr);
            if constexpr (NG == 2) {
                dma4(rs, dst, g0 & ~3u);
            } else if constexpr (NG == 4) {
                dma4(rs, dst, g0);
            } else {
                dma4(rs, dst, g0);
                dma4(rs, dst + 256, g0 + 4);
            }
        }
    } else if constexpr (ZP == kMetaPacked) {
        // the words of this lane's row stream from the one holding bit NG*kt*B on
        const uint32_t zo = lane * bf.zrow + 4 * (uint32_t)((NG * kt * B) >> 5);
#pragma unroll
        for (int e = 0; e < S::kZrOps; ++e) dma4(bf.zr, slot + S::kZr + 256 * e, zo + 4 * e);
        if constexpr (NG == 2) {
            dma4(bf.sc, slot + S::kSc, 2 * g0);
        } else if constexpr (NG == 4) {
            dma4(bf.sc, slot + S::kSc, 2 * g0);
            dma4(bf.sc, slot + S::kSc + 256, 2 * g0 + 4);
        } else {
            dma16(bf.sc, slot + S::kSc, 2 * g0);
        }
    } else if constexpr (NG == 2) {
        dma4(bf.sc, slot + S::kSc, 2 * g0);
        dma4(bf.zr, slot + S::kZr, g0 & ~3u);
    } else if constexpr (NG == 4) {
        dma4(bf.sc, slot + S::kSc, 2 * g0);
        dma4(bf.sc, slot + S::kSc + 256, 2 * g0 + 4);
        dma4(bf.zr, slot + S::kZr, g0);
    } else {
        dma16(bf.sc, slot + S::kSc, 2 * g0);
        dma4(bf.zr, slot + S::kZr, g0);
        dma4(bf.zr, slot + S::kZr + 256, g0 + 4);
    }
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-row block of problem p on this workgroup; slot0/slot1 are this wave's two ring slots
// (separate LDS arrays), `red` the workgroup's reduction buffer.
template <int B, int NW, int D, int MX, int GS, int ZP>
__device__ __forceinline__ void gemv_block(const GemvProblem &a, int64_t rb, uint8_t *slot0, uint8_t *slot1,
                                           f4 (*red)[64])
{
    static_assert(D == 2, "two ring slots");
    using S = RingSlot<B, MX, GS, ZP>;
    constexpr int NG = S::NG;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int64_t KT = a.k / kTileK, G = a.k / GS;

    GemvBufs bf;
    bf.G = G;
    bf.w = make_rsrc(a.w.packed + rb * KT * (512 * B), KT * (512 * B));
    if constexpr (ZP == kMetaFp8)
        bf.sc = make_rsrc((const uint8_t *)a.w.scales + rb * kTileN * G, kTileN * G);
    else
        bf.sc = make_rsrc(a.w.scales + rb * kTileN * G, kTileN * G * 2);
    if constexpr (ZP == kMetaPacked) {
        bf.zrow = (uint32_t)a.zrow;
        bf.zr = make_rsrc(a.w.zeros + rb * kTileN * a.zrow, kTileN * a.zrow);
    } else {
        bf.zrow = 0;
        bf.zr = make_rsrc(a.w.zeros + rb * kTileN * G, a.zmid ? 0 : kTileN * G);  // implied: none read
    }
    bf.x = make_rsrc(a.x, a.m * a.ldx * 2);  // rows >= m read as zeros

    const int64_t nt = KT > wv ? (KT - wv + NW - 1) / NW : 0;  // tiles of this wave
    ring_issue<B, MX, GS, ZP>(bf, wv, lane, a.ldx, slot0);

    // Activation fragments: lanes of rows >= m keep zeros and never read LDS.
    const bool act = r < a.m;
    h8 X[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) X[j] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
    f4 tot = {0.f, 0.f, 0.f, 0.f};
    float F[4] = {1.f, 1.f, 1.f, 1.f};  // fp8: the factors of rows 4t + i
    if constexpr (ZP == kMetaFp8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) F[i] = a.w.rowf[rb * kTileN + 4 * t + i];
    }
    // Tile i sits in slot i % 2 and the DMA of tile i+1 runs while tile i is consumed.  The two
    // slots are separate LDS arrays, named statically (the loop is unrolled by two), so the
    // compiler can tell that a slot's reads never overlap the DMA in flight into the other;
    // with one array and computed slot addresses it waits for every outstanding DMA before
    // each read, which serialises the loads with the arithmetic.
    for (int64_t i0 = 0; i0 < nt; i0 += 2)
#pragma unroll
    for (int sd = 0; sd < 2; ++sd) {
        const int64_t i = i0 + sd;
        if (i >= nt) break;  // uniform
        const int64_t kt = wv + i * NW;
        // At 2 and 4 bits nothing is fetched past the wave's last tile (2-2.5% faster at
        // 4096 x 4096); at 3, 5 and 6 bits the same branch measured 5-9% slower, so those widths
        // keep issuing the (out-of-range, zero-filled) fetch for the tile after the last.
        if ((B != 2 && B != 4) || i + 1 < nt) {  // uniform
            ring_issue<B, MX, GS, ZP>(bf, kt + NW, lane, a.ldx, sd == 0 ? slot1 : slot0);
            wait_vm<S::kLoads>();
        } else {
            wait_vm<0>();
        }
        const uint8_t *slot = sd == 0 ? slot0 : slot1;
        uint32_t d[2 * B];
#pragma unroll
        for (int sl = 0; sl < B / 2; ++sl) {
            const u4 v = *(const u4 *)(slot + 1024 * sl + 16 * lane);
            d[4 * sl + 0] = v[0];
            d[4 * sl + 1] = v[1];
            d[4 * sl + 2] = v[2];
            d[4 * sl + 3] = v[3];
        }
        if (B & 1) {
            d[2 * B - 2] = *(const uint32_t *)(slot + 1024 * (B / 2) + 4 * lane);
            d[2 * B - 1] = *(const uint32_t *)(slot + 1024 * (B / 2) + 256 + 4 * lane);
        }
        if (act) {
            const uint8_t *xb = slot + S::kX + 512 * r + 16 * t;
#pragma unroll
            for (int j = 0; j < 8; ++j) X[j] = *(const h8 *)(xb + 2 * (128 * (j >> 2) + 32 * (j & 3)));
        }
        // scales of rows 4t..4t+3 (two groups per word) and zero points of row r
        uint32_t sc[4][NG / 2];
        uint32_t zw[NG == 8 ? 2 : 1];
        float scf[4][NG];  // fp8: E4M3 values of rows 4t..4t+3
        if constexpr (ZP == kMetaFp8) {
            // scale bytes of row 4t+i: NG = 2 the pair inside the row's aligned word, else one
            // word (NG = 4) or two (NG = 8) per row
            uint32_t sw[4][NG == 8 ? 2 : 1];
            uint32_t esc = 0;
            if constexpr (NG == 2) {
                const u4 v = *(const u4 *)(slot + S::kSc + 16 * t);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t par = (uint32_t)(((4 * t + i) * G + 2 * kt) & 3);
                    sw[i][0] = (v[i] >> (8 * par)) & 0xFFFF;
                    esc |= sw[i][0];
                    e4m3_pair<false>(sw[i][0], scf[i][0], scf[i][1]);
                }
            } else {
#pragma unroll
                for (int h = 0; h < NG / 4; ++h) {
                    const u4 v = *(const u4 *)(slot + S::kSc + 256 * h + 16 * t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sw[i][h] = v[i];
                        esc |= v[i];
                        e4m3_pair<false>(v[i], scf[i][4 * h], scf[i][4 * h + 1]);
                        e4m3_pair<true>(v[i], scf[i][4 * h + 2], scf[i][4 * h + 3]);
                    }
                }
            }
            if (esc & 0x80808080u) {
                // a fallback group (rare): its fp16 scale from the row's list, divided by the
                // row factor that multiplies the row sum at the end; an index past the list
                // (malformed bytes) reads its last entry, or 0 for an empty list
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < NG; ++c) {
                        const uint32_t b = (sw[i][c / 4] >> (8 * (c % 4))) & 0xFF;
                        if (b & 0x80) {
                            const int j = min((int)(b & 0x7F), a.w.fb_stride - 1);
                            const int64_t row = rb * kTileN + 4 * t + i;
                            scf[i][c] = j >= 0 ? h_f(a.w.fb[row * a.w.fb_stride + j]) / F[i] : 0.0f;
                        }
                    }
            }
            const uint32_t zpar = (uint32_t)((r * G + NG * kt) & 3);
            if constexpr (NG == 2) zw[0] = *(const uint16_t *)(slot + S::kZr + 4 * r + zpar);
            else zw[0] = *(const uint32_t *)(slot + S::kZr + 4 * r);
            if constexpr (NG == 8) zw[1] = *(const uint32_t *)(slot + S::kZr + 256 + 4 * r);
        } else if constexpr (NG == 2) {
            const u4 v = *(const u4 *)(slot + S::kSc + 16 * t);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i][0] = v[i];
            if constexpr (ZP == kMetaByte) {
                const uint32_t zpar = (uint32_t)((r * G + 2 * kt) & 3);
                zw[0] = *(const uint16_t *)(slot + S::kZr + 4 * r + zpar);
            }
        } else if constexpr (NG == 4) {
            const u4 v0 = *(const u4 *)(slot + S::kSc + 16 * t), v1 = *(const u4 *)(slot + S::kSc + 256 + 16 * t);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i][0] = v0[i];
                sc[i][1] = v1[i];
            }
            if constexpr (ZP == kMetaByte) zw[0] = *(const uint32_t *)(slot + S::kZr + 4 * r);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u4 v = *(const u4 *)(slot + S::kSc + 16 * (4 * t + i));
                sc[i][0] = v[0];
                sc[i][1] = v[1];
                sc[i][2] = v[2];
                sc[i][3] = v[3];
            }
            if constexpr (ZP == kMetaByte) {
                zw[0] = *(const uint32_t *)(slot + S::kZr + 4 * r);
                zw[1] = *(const uint32_t *)(slot + S::kZr + 256 + 4 * r);
            }
        }
        GroupConst<B> gc[NG];
        if constexpr (ZP == kMetaPacked) {
            // fields c = 0 .. NG-1 at bits sh + c*B of the words fetched from the row stream
            uint32_t zp[3] = {0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < S::kZrOps; ++e) zp[e] = *(const uint32_t *)(slot + S::kZr + 256 * e + 4 * r);
            const uint64_t lo = zp[0] | ((uint64_t)zp[1] << 32), hi = zp[1] | ((uint64_t)zp[2] << 32);
            const int sh = (int)((NG * kt * B) & 31);
#pragma unroll
            for (int c = 0; c < NG; ++c) {
                const int p = sh + c * B;
                const uint32_t v = p < 32 ? (uint32_t)(lo >> p) : (uint32_t)(hi >> (p - 32));
                gc[c].set(v & ((1u << B) - 1));
            }
        } else {
#pragma unroll
            for (int c = 0; c < NG; ++c) gc[c].set(a.zmid ? (a.zmid & 0xFF) : (zw[c / 4] >> (8 * (c % 4))) & 0xFF);
        }
        h8 A[8];
        unpack_chunk_groups<B, NG>(d, gc, A);
        if constexpr (ZP == kMetaFp8)
            mma_tile_f<NG>(A, X, scf, tot);
        else
            mma_tile<NG>(A, X, sc, tot);
    }
    wait_vm<0>();  // drain the tiles issued past the end before the workgroup's LDS is released

    red[wv][lane] = tot;
    __syncthreads();
    if (wv != 0 || r >= a.m) return;
    f4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[w][lane];
    if constexpr (ZP == kMetaFp8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] *= F[i];
    }
    if (a.rowptr) {
        const uint16_t *xrow = a.x + r * a.ldx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = rb * kTileN + 4 * t + i;
            for (int32_t p = a.rowptr[n]; p < a.rowptr[n + 1]; ++p)
                s[i] = __builtin_fmaf(h_f(xrow[a.col[p]]), h_f(a.val[p]), s[i]);
        }
    }
    uint16_t *y = a.y + r * a.ldy + rb * kTileN + 4 * t;
    *(u2 *)y = (u2){pack_h2(s[0], s[1]), pack_h2(s[2], s[3])};
}

// One problem, one workgroup per 16-row block.
template <int B, int NW, int D, int MX, int GS, int ZP>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(GemvProblem a)
{
    constexpr int pitch = RingSlot<B, MX, GS, ZP>::kBytes;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[NW][pitch];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[NW][pitch];
    __shared__ f4 red[NW][64];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    gemv_block<B, NW, D, MX, GS, ZP>(a, blockIdx.x, &ring0[wv][0], &ring1[wv][0], red);
}

// Independent problems (mixed bit widths up to BM, one group size) in one launch: workgroup b
// serves problem p with block0 <= b < block0 + n/16.  The ring slots are sized for BM-bit tiles
// (smaller slots leave LDS for more workgroups per CU).
template <int NW, int D, int MX, int GS, int ZP, int BM>
__global__ __launch_bounds__(NW * 64) void gemv_batch_kernel(GemvBatch bt)
{
    constexpr int pitch = RingSlot<BM, MX, GS, ZP>::kBytes;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[NW][pitch];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[NW][pitch];
    __shared__ f4 red[NW][64];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxGemvBatch; ++i)
        if (i < bt.count && b >= bt.p[i].block0) p = i;
    const GemvProblem &a = bt.p[p];
    const int64_t rb = b - a.block0;
    uint8_t *s0 = &ring0[wv][0], *s1 = &ring1[wv][0];
    switch (a.bits) {
    case 2: gemv_block<2, NW, D, MX, GS, ZP>(a, rb, s0, s1, red); break;
    case 3:
        if constexpr (BM >= 3) gemv_block<3, NW, D, MX, GS, ZP>(a, rb, s0, s1, red);
        break;
    case 4:
        if constexpr (BM >= 4) gemv_block<4, NW, D, MX, GS, ZP>(a, rb, s0, s1, red);
        break;
    case 5:
        if constexpr (BM >= 5) gemv_block<5, NW, D, MX, GS, ZP>(a, rb, s0, s1, red);
        break;
    default:
        if constexpr (BM >= 6) gemv_block<6, NW, D, MX, GS, ZP>(a, rb, s0, s1, red);
        break;
    }
}

template <int B, int MX, int GS, int ZP>
static hipError_t gemv_mx(const GemvProblem &a, hipStream_t st)
{
    // Wide matrices have row blocks enough to fill the GPU with 4-wave workgroups (more of
    // them fit per CU); narrow ones split each row block's k over 8 waves.
    // (Eight waves with an 8-row-pair activation ring would exceed the 160 KB of LDS.)
    const int64_t blocks = a.n / kTileN;
    if constexpr (MX == 8) {
        hipLaunchKernelGGL((gemv_kernel<B, 4, 2, MX, GS, ZP>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    } else {
        if (blocks >= 512)
            hipLaunchKernelGGL((gemv_kernel<B, 4, 2, MX, GS, ZP>), dim3((unsigned)blocks), dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((gemv_kernel<B, 8, 2, MX, GS, ZP>), dim3((unsigned)blocks), dim3(512), 0, st, a);
    }
    return hipGetLastError();
}

template <int B, int GS, int ZP>
static hipError_t gemv_bits_gs(const GemvProblem &a, hipStream_t st)
{
    if (a.m <= 2) return gemv_mx<B, 1, GS, ZP>(a, st);
    if (a.m <= 4) return gemv_mx<B, 2, GS, ZP>(a, st);
    if (a.m <= 8) return gemv_mx<B, 4, GS, ZP>(a, st);
    return gemv_mx<B, 8, GS, ZP>(a, st);
}
template <int B, int ZP>
static hipError_t gemv_bits(const GemvProblem &a, hipStream_t st)
{
    if (a.gs == 32) return gemv_bits_gs<B, 32, ZP>(a, st);
    if (a.gs == 64) return gemv_bits_gs<B, 64, ZP>(a, st);
    return gemv_bits_gs<B, 128, ZP>(a, st);
}

template <int ZP>
static hipError_t gemv_zp(const GemvProblem &a, hipStream_t st)
{
    switch (a.bits) {
    case 2: return gemv_bits<2, ZP>(a, st);
    case 3: return gemv_bits<3, ZP>(a, st);
    case 4: return gemv_bits<4, ZP>(a, st);
    case 5: return gemv_bits<5, ZP>(a, st);
    case 6: return gemv_bits<6, ZP>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvProblem &a, hipStream_t st)
{
    if (a.fp8) return gemv_zp<kMetaFp8>(a, st);
    return a.zrow ? gemv_zp<kMetaPacked>(a, st) : gemv_zp<kMetaByte>(a, st);
}

template <int MX, int GS, int ZP, int BM>
static hipError_t gemv_batch_mx(const GemvBatch &b, int64_t blocks, hipStream_t st)
{
    if constexpr (MX >= 4) {
        hipLaunchKernelGGL((gemv_batch_kernel<4, 2, MX, GS, ZP, BM>), dim3((unsigned)blocks), dim3(256), 0, st, b);
    } else {
        if (blocks >= 512)
            hipLaunchKernelGGL((gemv_batch_kernel<4, 2, MX, GS, ZP, BM>), dim3((unsigned)blocks), dim3(256), 0, st, b);
        else
            hipLaunchKernelGGL((gemv_batch_kernel<8, 2, MX, GS, ZP, BM>), dim3((unsigned)blocks), dim3(512), 0, st, b);
    }
    return hipGetLastError();
}

template <int GS, int ZP, int BM>
static hipError_t gemv_batch_gs(const GemvBatch &b, int64_t blocks, int m_max, hipStream_t st)
{
    if (m_max <= 2) return gemv_batch_mx<1, GS, ZP, BM>(b, blocks, st);
    if (m_max <= 4) return gemv_batch_mx<2, GS, ZP, BM>(b, blocks, st);
    if (m_max <= 8) return gemv_batch_mx<4, GS, ZP, BM>(b, blocks, st);
    return gemv_batch_mx<8, GS, ZP, BM>(b, blocks, st);
}

template <int ZP, int BM>
static hipError_t gemv_batch_zp(const GemvBatch &b, int64_t blocks, int m_max, hipStream_t st)
{
    if (b.p[0].gs == 32) return gemv_batch_gs<32, ZP, BM>(b, blocks, m_max, st);
    if (b.p[0].gs == 64) return gemv_batch_gs<64, ZP, BM>(b, blocks, m_max, st);
    return gemv_batch_gs<128, ZP, BM>(b, blocks, m_max, st);
}

template <int BM>
static hipError_t gemv_batch_bm(const GemvBatch &b, int64_t blocks, int m_max, hipStream_t st)
{
    if (b.p[0].fp8) return gemv_batch_zp<kMetaFp8, BM>(b, blocks, m_max, st);
    return b.p[0].zrow ? gemv_batch_zp<kMetaPacked, BM>(b, blocks, m_max, st)
                       : gemv_batch_zp<kMetaByte, BM>(b, blocks, m_max, st);
}

// Ring slots sized for the widest problem of the batch: 2, 4 or 6 bits.
hipError_t launch_gemv_batch(const GemvBatch &b, int64_t blocks, int m_max, hipStream_t st)
{
    int bm = 2;
    for (int i = 0; i < b.count; ++i) bm = b.p[i].bits > bm ? b.p[i].bits : bm;
    if (bm <= 2) return gemv_batch_bm<2>(b, blocks, m_max, st);
    if (bm <= 4) return gemv_batch_bm<4>(b, blocks, m_max, st);
    return gemv_batch_bm<6>(b, blocks, m_max, st);
}

}  // namespace qp
