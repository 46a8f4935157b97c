// Quantized KV cache on gfx950: the write path (new K/V rows quantized into the cache) and
// decode attention that reads the packed codes and their scales directly.
//
// KV-cache quantization page (kwkr.cn): s2.1 symmetric groups, scale from the absolute
// maximum; s2.2 groups of adjacent head-dimension elements (32, 64 or 128); s2.3 K and V at
// their own bit widths (INT4 K with INT8 V); s3.1 one FP32 scale per group; s5.1 4-bit values
// two per byte and an attention operator that dequantizes in registers instead of writing an
// fp16 copy of the cache.  Head dimension 128.  This file is compiled without floating-point
// contraction so the write path is bit-identical to the CPU reference; the attention writes
// its fused multiply-adds explicitly.
//
// Cache storage (values counted in the tensor's own width; a 4-bit value p is the low nibble
// of byte p/2 when p is even):
//   sigma(s) = s (8-bit) or s/2 + 4*(s%2) (4-bit) places slot s = 0..7 of an 8-value piece.
//   K: row R = (b*Hkv + h)*cap + token, 128*kb/8 bytes; value d = 32j + 8t + s at
//      32t + 8j + sigma(s).  Lane l = 16t + r of a wave reads token r's 16 (32) contiguous
//      bytes at 16t (32t): the A operands of the four 16x16x32 matrix-core steps j.
//   V: per (b, h), tiles of 32 tokens (32*128*vb/8 bytes); token w of a tile with
//      w = 4t + s (s < 4) or 16 + 4t + s - 4 (s >= 4) and value d = 16c + r belong to lane
//      l = 16t + r, slice c (its eight tokens at one d: the A operand of V^T), slot s.  The
//      lane's slices fill 16-byte pieces of P = 128/vb values, and piece e of lane l sits at
//      64*P*e + P*l, so each of the tile's 16-byte fetches reads 1 KB contiguous.
//   Scales: fp32 [R][128/g].
//
// Attention (one query token per sequence, GQA: query head h reads kv head h / (Hq/Hkv)):
// a workgroup of four waves takes one (sequence, kv head, token chunk); each wave walks its
// 32-token tiles with an online softmax for all query heads of the kv head at once (up to 16,
// the matrix-core N dimension; missing heads are zero columns).
//   scores:  S^T[token][head] = K codes (exact fp16 integers) x Q^T per group of the head
//            dimension, each group scaled by its fp32 K scale in fp32.  Lane (t, r) receives
//            the scores of tokens 4t+i and 16+4t+i (i = 0..3) for head r -- exactly the eight
//            tokens it supplies to the V product below, so no value crosses lanes except the
//            row maximum.
//   softmax: base-2 exponent with the log2(e) factor folded into the score scale; weights
//            exp2(z - m + 14) <= 2^14 so fp16 keeps them normal far below the maximum; the
//            2^14 cancels in o / l.
//   values:  O^T[d][head] += (V codes * V scale, rounded to fp16) x P^T on the matrix core.
// The four waves' (m, l, O) are merged through LDS; with several chunks per (sequence, kv
// head) the partial results go to the workspace and a second kernel merges them.
#include "bufio.h"
#include "kv_internal.h"
#include "unpack.h"

namespace qp {

constexpr int kD = 128;

// ---- storage maps ------------------------------------------------------------------------

__device__ __forceinline__ int kv_sigma(int bits, int s) { return bits == 8 ? s : s / 2 + 4 * (s % 2); }

__device__ __forceinline__ int kv_k_pos(int bits, int d)
{
    return 32 * ((d % 32) / 8) + 8 * (d / 32) + kv_sigma(bits, d % 8);
}

__device__ __forceinline__ int kv_v_pos(int bits, int w, int d)
{
    const int hi = w >= 16, t = (w % 16) / 4, s = (w % 4) + 4 * hi;
    const int c = d / 16, l = 16 * t + d % 16, P = 128 / bits, spp = P / 8;
    return 64 * P * (c / spp) + P * l + 8 * (c % spp) + kv_sigma(bits, s);
}

// ---- write path: one wave per row, lane l holds d = l and d = 64 + l ---------------------

template <int BITS, int WHICH, int G>
__global__ __launch_bounds__(256) void kv_quantize_kernel(KvQuantArgs a)
{
    constexpr int qmax = (1 << (BITS - 1)) - 1, mid = 1 << (BITS - 1), NG = kD / G;
    constexpr int span = G < 64 ? G : 64;
    __shared__ uint8_t stage[4][kD];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wv;
    const bool in = row < a.rows;
    const int64_t slot = in ? a.slots[row] : -1;
    const bool ok = in && slot >= 0 && slot < a.total_rows;
    float v[2] = {0.f, 0.f};
    if (ok) {
        const uint16_t *x = a.x + row * a.ldx;
        v[0] = h_f(x[lane]);
        v[1] = h_f(x[64 + lane]);
    }
    float m[2] = {__builtin_fabsf(v[0]), __builtin_fabsf(v[1])};
#pragma unroll
    for (int off = span / 2; off >= 1; off >>= 1) {
        m[0] = __builtin_fmaxf(m[0], __shfl_xor(m[0], off));
        m[1] = __builtin_fmaxf(m[1], __shfl_xor(m[1], off));
    }
    if constexpr (G == 128) m[0] = m[1] = __builtin_fmaxf(m[0], m[1]);
    uint8_t c[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float s = m[e] / (float)qmax;
        int q = 0;
        if (m[e] != 0.f) {
            q = (int)__builtin_rintf(v[e] / s);
            q = q < -qmax ? -qmax : (q > qmax ? qmax : q);
        }
        c[e] = (uint8_t)(q + mid);
        const int d = 64 * e + lane;
        if (ok && d % G == 0) a.scales[slot * NG + d / G] = m[e] == 0.f ? 0.f : s;
    }
    if constexpr (WHICH == 0 && BITS == 4) {
        // A K row's nibbles all belong to this row: gather whole bytes through LDS.
        stage[wv][lane] = c[0];
        stage[wv][64 + lane] = c[1];
        __syncthreads();
        if (ok) {
            // byte l holds nibble positions 2l, 2l + 1; position p = 32t + 8j + sigma(s)
            uint32_t byte = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int p = 2 * lane + h, t = p / 32, j = (p % 32) / 8, sg = p % 8;
                const int s = sg < 4 ? 2 * sg : 2 * (sg - 4) + 1;
                byte |= (uint32_t)stage[wv][32 * j + 8 * t + s] << (4 * h);
            }
            a.codes[slot * (kD / 2) + lane] = (uint8_t)byte;
        }
    } else if (ok) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d = 64 * e + lane;
            int64_t pos;
            if constexpr (WHICH == 0) {
                pos = slot * kD + kv_k_pos(BITS, d);
            } else {
                const int64_t region = slot / a.cap, tau = slot % a.cap;
                pos = (region * a.cap + (tau / 32) * 32) * kD + kv_v_pos(BITS, (int)(tau % 32), d);
            }
            if constexpr (BITS == 8) {
                a.codes[pos] = c[e];
            } else {
                // Two tokens share each byte of a V tile: replace only this nibble.
                uint32_t *wd = (uint32_t *)a.codes + pos / 8;
                const int sh = 4 * (int)(pos % 8);
                atomicAnd(wd, ~(0xFu << sh));
                atomicOr(wd, (uint32_t)c[e] << sh);
            }
        }
    }
}

template <int BITS, int WHICH>
static hipError_t quant_g(const KvQuantArgs &a, int g, hipStream_t st)
{
    const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
    if (g == 32) hipLaunchKernelGGL((kv_quantize_kernel<BITS, WHICH, 32>), grid, block, 0, st, a);
    else if (g == 64) hipLaunchKernelGGL((kv_quantize_kernel<BITS, WHICH, 64>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kv_quantize_kernel<BITS, WHICH, 128>), grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv_quantize(int bits, int which, int g, const KvQuantArgs &a, hipStream_t st)
{
    if (a.rows == 0) return hipSuccess;
    if (bits == 4) return which == 0 ? quant_g<4, 0>(a, g, st) : quant_g<4, 1>(a, g, st);
    return which == 0 ? quant_g<8, 0>(a, g, st) : quant_g<8, 1>(a, g, st);
}

// ---- decode attention ---------------------------------------------------------------------

// Eight offset 4-bit codes of one piece (sigma order) -> the eight signed values, slot order.
__device__ __forceinline__ h8 unpack_nib8(uint32_t w)
{
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f}, sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 a0 = {(_Float16)-1032.0f, (_Float16)-1032.0f}, a1 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t p0 = magic_pair<0x000F000Fu>(w, one, a0);        // slots 0, 1
    const uint32_t p1 = magic_pair<0x00F000F0u>(w, sixteenth, a1);  // slots 2, 3
    const uint32_t w8 = w >> 8;
    const uint32_t p2 = magic_pair<0x000F000Fu>(w8, one, a0);       // slots 4, 5
    const uint32_t p3 = magic_pair<0x00F000F0u>(w8, sixteenth, a1); // slots 6, 7
    const u4 r = {p0, p1, p2, p3};
    return __builtin_bit_cast(h8, r);
}

// Eight offset 8-bit codes (slot order) -> the eight signed values.  v_perm_b32 places code
// bytes under the 0x64 exponent byte (1024 + code in each half) in one step per pair.
__device__ __forceinline__ h8 unpack_byte8(uint32_t w0, uint32_t w1)
{
    const h2 a = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t hi = 0x64646464u;
    u4 r;
    r[0] = h2_bits(bits_h2(__builtin_amdgcn_perm(hi, w0, 0x04010400u)) + a);  // bytes 0, 1
    r[1] = h2_bits(bits_h2(__builtin_amdgcn_perm(hi, w0, 0x04030402u)) + a);  // bytes 2, 3
    r[2] = h2_bits(bits_h2(__builtin_amdgcn_perm(hi, w1, 0x04010400u)) + a);
    r[3] = h2_bits(bits_h2(__builtin_amdgcn_perm(hi, w1, 0x04030402u)) + a);
    return __builtin_bit_cast(h8, r);
}

// A wave's ring slot: one 32-token tile.  Code pieces are fetched by 16-byte buffer-to-LDS
// DMA, lane l's piece landing at 16*l of a 1 KB block, so each lane later reads back exactly
// the bytes it fetched; the tile's fp32 K and V scales (token-major, 32*G floats) come by
// 4-byte DMA.  Bytes in flight cost no registers, so a wave keeps D-1 tiles in flight.
template <int KB, int VB, int GK, int GV>
struct KvSlot {
    static constexpr int kK = 0;                        // K: u = 0, 1 (16 tokens each) x KB/4 blocks
    static constexpr int kV = kK + 1024 * (KB / 2);     // V: VB/2 blocks
    static constexpr int kKsOps = GK > 2 ? GK / 2 : 1;  // 256-byte DMAs of K scales
    static constexpr int kVsOps = GV > 2 ? GV / 2 : 1;
    static constexpr int kKs = kV + 1024 * (VB / 2);
    static constexpr int kVs = kKs + 256 * kKsOps;
    static constexpr int kBytes = kVs + 256 * kVsOps;
    static constexpr int kLoads = KB / 2 + VB / 2 + kKsOps + kVsOps;  // DMA instructions per tile
};

constexpr int kKvWaves = 4, kKvDepth = 2;

struct KvBufs {
    rsrc_t k, ks, v, vs;
};

__device__ __forceinline__ void kv_dma16(rsrc_t r, uint8_t *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void kv_dma4(rsrc_t r, uint8_t *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

// Fetch tile T into a slot.  Tiles past the sequence read zeros (buffer range) and tiles past
// the wave's share are fetched but never read, so every step issues the same DMA count.
template <int KB, int VB, int GK, int GV>
__device__ __forceinline__ void kv_issue(const KvBufs &bf, int T, int lane, uint8_t *slot)
{
    using S = KvSlot<KB, VB, GK, GV>;
    constexpr int KRB = kD * KB / 8, VTB = 32 * kD * VB / 8;
    const int t = lane >> 4, r = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < KB / 4; ++e)
            kv_dma16(bf.k, slot + S::kK + 1024 * (u * (KB / 4) + e),
                     (uint32_t)((32 * T + 16 * u + r) * KRB + (KRB / 4) * t + 16 * e));
#pragma unroll
    for (int e = 0; e < VB / 2; ++e)
        kv_dma16(bf.v, slot + S::kV + 1024 * e, (uint32_t)(T * VTB + 1024 * e + 16 * lane));
#pragma unroll
    for (int e = 0; e < S::kKsOps; ++e)
        kv_dma4(bf.ks, slot + S::kKs + 256 * e, (uint32_t)(32 * T * GK * 4 + 256 * e + 4 * lane));
#pragma unroll
    for (int e = 0; e < S::kVsOps; ++e)
        kv_dma4(bf.vs, slot + S::kVs + 256 * e, (uint32_t)(32 * T * GV * 4 + 256 * e + 4 * lane));
}

template <int N>
__device__ __forceinline__ void kv_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int KB>
__device__ __forceinline__ h8 k_frag(const u4 (&k)[KB / 4], int j)
{
    if constexpr (KB == 4) return unpack_nib8(k[0][j]);
    else return unpack_byte8(k[j / 2][(2 * j) % 4], k[j / 2][(2 * j) % 4 + 1]);
}

template <int VB>
__device__ __forceinline__ h8 v_frag(const u4 (&v)[VB / 2], int c)
{
    if constexpr (VB == 4) return unpack_nib8(v[c / 4][c % 4]);
    else return unpack_byte8(v[c / 2][(2 * c) % 4], v[c / 2][(2 * c) % 4 + 1]);
}

// max(v[l], v[l ^ X]) for X = 16 or 32 without a trip through LDS: the gfx950 permlane swaps
// exchange 16-lane rows (odd with even) or the two 32-lane halves, so the pair of results
// holds both values at every lane.
template <int X>
__device__ __forceinline__ float max_pair(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    uint32_t a, b;
    if constexpr (X == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        a = r[0];
        b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        a = r[0];
        b = r[1];
    }
    return __builtin_fmaxf(as_f(a), as_f(b));
}

// Online-softmax state of a wave: running maximum m (base 2, shared by the four lanes of a
// head), the lane's share l of the weight sum, and O^T (lane (t, r): d = 16c + 4t + i, head r).
struct KvState {
    float m, l;
    f4 O[8];
};

// Consume tile T from a slot: scores, softmax update, values.
template <int KB, int VB, int KG, int VG>
__device__ __forceinline__ void kv_tile(const uint8_t *slot, int T, int t1, const h8 (&Q)[4], float c, int lane,
                                        KvState &st)
{
    constexpr int GK = kD / KG, GV = kD / VG, KSTEP = KG / 32;
    using S = KvSlot<KB, VB, GK, GV>;
    const int t = lane >> 4;
    u4 kd[2][KB / 4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < KB / 4; ++e) kd[u][e] = *(const u4 *)(slot + S::kK + 1024 * (u * (KB / 4) + e) + 16 * lane);
    u4 vd[VB / 2];
#pragma unroll
    for (int e = 0; e < VB / 2; ++e) vd[e] = *(const u4 *)(slot + S::kV + 1024 * e + 16 * lane);
    float ks[2][4 * GK], vs[2][4 * GV];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < GK; ++e) {
            const u4 v = *(const u4 *)(slot + S::kKs + ((16 * u + 4 * t) * GK + 4 * e) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) ks[u][4 * e + i] = as_f(v[i]);
        }
#pragma unroll
        for (int e = 0; e < GV; ++e) {
            const u4 v = *(const u4 *)(slot + S::kVs + ((16 * u + 4 * t) * GV + 4 * e) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) vs[u][4 * e + i] = as_f(v[i]);
        }
    }
    // scores of tokens 32T + 16u + 4t + i for head r, in base-2 units
    float z[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        f4 zt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < GK; ++gi) {
            f4 acc = mfma16(k_frag<KB>(kd[u], KSTEP * gi), Q[KSTEP * gi], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int jj = 1; jj < KSTEP; ++jj) acc = mfma16(k_frag<KB>(kd[u], KSTEP * gi + jj), Q[KSTEP * gi + jj], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) zt[i] = __builtin_fmaf(ks[u][GK * i + gi], acc[i], zt[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) z[u][i] = zt[i] * c;
    }
    if (32 * T + 32 > t1) {  // the sequence or chunk ends inside this tile (wave-uniform)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (32 * T + 16 * (e / 4) + 4 * t + e % 4 >= t1) z[e / 4][e % 4] = -__builtin_inff();
    }
    float mt = z[0][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = __builtin_fmaxf(mt, z[e / 4][e % 4]);
    mt = max_pair<16>(mt);
    mt = max_pair<32>(mt);
    const float mn = __builtin_fmaxf(st.m, mt);  // finite: token 32T < t1 is in every tile
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    const float base = mn - 14.0f;
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(z[e / 4][e % 4] - base);
        ps += p[e];
    }
    st.l = __builtin_fmaf(st.l, alpha, ps);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st.O[cc] *= alpha;
    }
    const u4 pw = {pack_h2(p[0], p[1]), pack_h2(p[2], p[3]), pack_h2(p[4], p[5]), pack_h2(p[6], p[7])};
    const h8 P = __builtin_bit_cast(h8, pw);
    h8 vsh[GV];
#pragma unroll
    for (int gi = 0; gi < GV; ++gi) {
        const u4 w = {pack_h2(vs[0][GV * 0 + gi], vs[0][GV * 1 + gi]), pack_h2(vs[0][GV * 2 + gi], vs[0][GV * 3 + gi]),
                      pack_h2(vs[1][GV * 0 + gi], vs[1][GV * 1 + gi]), pack_h2(vs[1][GV * 2 + gi], vs[1][GV * 3 + gi])};
        vsh[gi] = __builtin_bit_cast(h8, w);
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        const h8 vq = v_frag<VB>(vd, cc) * vsh[(16 * cc) / VG];
        st.O[cc] = mfma16(vq, P, st.O[cc]);
    }
}

// A wave's tiles i = 0 .. nt-1 (tile T0 + i*kKvWaves) through its ring of kKvDepth slots.
// The slots are restrict pointers and the loop is unrolled by the depth, so every slot access
// names a slot statically and the compiler never waits for a DMA in flight into another slot.
template <int KB, int VB, int KG, int VG>
__device__ __forceinline__ void kv_loop(const KvBufs &bf, uint8_t *__restrict__ s0, uint8_t *__restrict__ s1,
                                        uint8_t *__restrict__ s2, int T0, int nt, int t1, const h8 (&Q)[4], float c,
                                        int lane, KvState &st)
{
    constexpr int GK = kD / KG, GV = kD / VG, W = kKvWaves, D = kKvDepth;
    using S = KvSlot<KB, VB, GK, GV>;
    static_assert(D == 2 || D == 3, "two or three slots");
    kv_issue<KB, VB, GK, GV>(bf, T0, lane, s0);
    if constexpr (D == 3) {
        kv_issue<KB, VB, GK, GV>(bf, T0 + W, lane, s1);
        for (int i = 0; i < nt; i += 3) {
            kv_issue<KB, VB, GK, GV>(bf, T0 + W * (i + 2), lane, s2);
            kv_wait_vm<2 * S::kLoads>();
            kv_tile<KB, VB, KG, VG>(s0, T0 + W * i, t1, Q, c, lane, st);
            if (i + 1 >= nt) break;
            kv_issue<KB, VB, GK, GV>(bf, T0 + W * (i + 3), lane, s0);
            kv_wait_vm<2 * S::kLoads>();
            kv_tile<KB, VB, KG, VG>(s1, T0 + W * (i + 1), t1, Q, c, lane, st);
            if (i + 2 >= nt) break;
            kv_issue<KB, VB, GK, GV>(bf, T0 + W * (i + 4), lane, s1);
            kv_wait_vm<2 * S::kLoads>();
            kv_tile<KB, VB, KG, VG>(s2, T0 + W * (i + 2), t1, Q, c, lane, st);
        }
    } else {
        (void)s2;
        for (int i = 0; i < nt; i += 2) {
            kv_issue<KB, VB, GK, GV>(bf, T0 + W * (i + 1), lane, s1);
            kv_wait_vm<S::kLoads>();
            kv_tile<KB, VB, KG, VG>(s0, T0 + W * i, t1, Q, c, lane, st);
            if (i + 1 >= nt) break;
            kv_issue<KB, VB, GK, GV>(bf, T0 + W * (i + 2), lane, s0);
            kv_wait_vm<S::kLoads>();
            kv_tile<KB, VB, KG, VG>(s1, T0 + W * (i + 1), t1, Q, c, lane, st);
        }
    }
    kv_wait_vm<0>();  // drain the fetches past the end before the LDS is reused
}

template <int KB, int VB, int KG, int VG>
__global__ __launch_bounds__(kKvWaves * 64) void kv_attn_kernel(KvAttnArgs a)
{
    constexpr int GK = kD / KG, GV = kD / VG, W = kKvWaves;
    constexpr int KRB = kD * KB / 8, VTB = 32 * kD * VB / 8;
    constexpr int pitch = KvSlot<KB, VB, GK, GV>::kBytes;
    constexpr int ring_bytes = kKvDepth * W * pitch, merge_bytes = W * 16 * (kD + 1) * 4;
    __shared__ __attribute__((aligned(16))) uint8_t ring[ring_bytes > merge_bytes ? ring_bytes : merge_bytes];
    __shared__ float sm_m[W][16], sm_l[W][16];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane >> 4, r = lane & 15;
    const int b = blockIdx.z, hk = blockIdx.y, sp = blockIdx.x;
    int L = a.lens[b];
    L = L < 0 ? 0 : (L > a.cap ? (int)a.cap : L);
    const int t0 = sp * a.chunk, t1 = t0 + a.chunk < L ? t0 + a.chunk : L;
    const int64_t R0 = ((int64_t)b * a.hkv + hk) * a.cap;
    KvBufs bf;
    bf.k = make_rsrc(a.kc + R0 * KRB, (int64_t)L * KRB);
    bf.ks = make_rsrc(a.ks + R0 * GK, (int64_t)L * GK * 4);
    bf.v = make_rsrc(a.vc + R0 * (kD * VB / 8), (int64_t)((L + 31) / 32) * VTB);
    bf.vs = make_rsrc(a.vs + R0 * GV, (int64_t)L * GV * 4);

    // B operand of the score product: head r's values d = 32j + 8t + s (zero past the group)
    h8 Q[4];
    const int64_t qrow = (int64_t)b * a.hq + (int64_t)hk * a.grp + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (r < a.grp) Q[j] = *(const h8 *)(a.q + qrow * kD + 32 * j + 8 * t);
        else Q[j] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
    }

    KvState st;
    st.m = -__builtin_inff();
    st.l = 0.f;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) st.O[cc] = (f4){0.f, 0.f, 0.f, 0.f};
    const int T0 = t0 / 32, ntiles = t1 > t0 ? (t1 + 31) / 32 - T0 : 0;
    const int nt = ntiles > wv ? (ntiles - wv + W - 1) / W : 0;
    if (nt > 0) {
        uint8_t *base = ring + (size_t)wv * kKvDepth * pitch;
        kv_loop<KB, VB, KG, VG>(bf, base, base + pitch, base + (kKvDepth - 1) * pitch, T0 + wv, nt, t1, Q, a.c,
                                lane, st);
    }
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    __syncthreads();  // every wave is done with its ring: the merge buffer overlays it
    float(*sm_o)[16][kD + 1] = reinterpret_cast<float(*)[16][kD + 1]>(ring);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_o[wv][r][16 * cc + 4 * t + i] = st.O[cc][i];
    if (t == 0) {
        sm_m[wv][r] = st.m;
        sm_l[wv][r] = st.l;
    }
    __syncthreads();
    const int64_t bh0 = (int64_t)b * a.hq + (int64_t)hk * a.grp;
    for (int idx = threadIdx.x; idx < a.grp * kD; idx += W * 64) {
        const int h = idx / kD, d = idx % kD;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < W; ++w) M = __builtin_fmaxf(M, sm_m[w][h]);
        float o = 0.f, S = 0.f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float e = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
                o = __builtin_fmaf(e, sm_o[w][h][d], o);
                S = __builtin_fmaf(e, sm_l[w][h], S);
            }
        }
        if (a.nsplit == 1) {
            const float y = S > 0.f ? o / S : 0.f;
            a.o[(bh0 + h) * kD + d] = __builtin_bit_cast(uint16_t, (_Float16)y);
        } else {
            const int64_t pi = (bh0 + h) * a.nsplit + sp;
            a.part_o[pi * kD + d] = o;
            if (d == 0) {
                a.part_ml[2 * pi] = M;
                a.part_ml[2 * pi + 1] = S;
            }
        }
    }
}

// Merge the chunks of one (sequence, query head): one thread per d.  The merge is bound by
// memory latency, so the partial outputs of the first kKvPre chunks are loaded together with
// the chunk maxima and sums, before anything depends on them; the maxima and sums are read
// once into LDS by all threads together, the maximum is reduced by wave shuffles, and the
// partial outputs of further chunks are read eight at a time.
constexpr int kKvMaxSplit = 1024;
constexpr int kKvPre = 16;

__global__ __launch_bounds__(kD) void kv_combine_kernel(KvAttnArgs a)
{
    __shared__ float sm_e[kKvMaxSplit], sm_s[kKvMaxSplit], red[kD / 64];
    const int64_t bh = blockIdx.x;
    const int d = threadIdx.x, ns = a.nsplit;
    const float *ml = a.part_ml + 2 * bh * ns;
    const float *po = a.part_o + bh * ns * kD + d;
    float pre[kKvPre];
#pragma unroll
    for (int i = 0; i < kKvPre; ++i) pre[i] = i < ns ? po[(int64_t)i * kD] : 0.f;
    float M = -__builtin_inff();
    for (int s = d; s < ns; s += kD) {
        const float m = ml[2 * s];
        sm_e[s] = m;
        sm_s[s] = ml[2 * s + 1];
        M = __builtin_fmaxf(M, m);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, off));
    if ((d & 63) == 0) red[d >> 6] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < kD / 64; ++w) M = __builtin_fmaxf(M, red[w]);
    float y = 0.f;
    if (M != -__builtin_inff()) {
        for (int s = d; s < ns; s += kD) sm_e[s] = __builtin_amdgcn_exp2f(sm_e[s] - M);
        __syncthreads();
        float o = 0.f, S = 0.f;
#pragma unroll
        for (int i = 0; i < kKvPre; ++i) {
            if (i < ns) {
                o = __builtin_fmaf(sm_e[i], pre[i], o);
                S = __builtin_fmaf(sm_e[i], sm_s[i], S);
            }
        }
        int s = kKvPre;
        for (; s + 8 <= ns; s += 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = po[(int64_t)(s + i) * kD];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o = __builtin_fmaf(sm_e[s + i], v[i], o);
                S = __builtin_fmaf(sm_e[s + i], sm_s[s + i], S);
            }
        }
        for (; s < ns; ++s) {
            o = __builtin_fmaf(sm_e[s], po[(int64_t)s * kD], o);
            S = __builtin_fmaf(sm_e[s], sm_s[s], S);
        }
        y = S > 0.f ? o / S : 0.f;
    }
    a.o[bh * kD + d] = __builtin_bit_cast(uint16_t, (_Float16)y);
}

template <int KB, int VB>
static hipError_t attn_kv(const KvAttnArgs &a, int kg, int vg, dim3 grid, hipStream_t st)
{
#define QP_KV_ATTN(KG, VG) \
    if (kg == KG && vg == VG) { hipLaunchKernelGGL((kv_attn_kernel<KB, VB, KG, VG>), grid, dim3(kKvWaves * 64), 0, st, a); return hipGetLastError(); }
    QP_KV_ATTN(32, 32) QP_KV_ATTN(32, 64) QP_KV_ATTN(32, 128)
    QP_KV_ATTN(64, 32) QP_KV_ATTN(64, 64) QP_KV_ATTN(64, 128)
    QP_KV_ATTN(128, 32) QP_KV_ATTN(128, 64) QP_KV_ATTN(128, 128)
#undef QP_KV_ATTN
    return hipErrorInvalidValue;
}

hipError_t launch_kv_attn(int kb, int vb, int kg, int vg, int64_t batch, const KvAttnArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)a.nsplit, (unsigned)a.hkv, (unsigned)batch);
    hipError_t e;
    if (kb == 4) e = vb == 4 ? attn_kv<4, 4>(a, kg, vg, grid, st) : attn_kv<4, 8>(a, kg, vg, grid, st);
    else e = vb == 4 ? attn_kv<8, 4>(a, kg, vg, grid, st) : attn_kv<8, 8>(a, kg, vg, grid, st);
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(kv_combine_kernel, dim3((unsigned)(batch * a.hq)), dim3(kD), 0, st, a);
    return hipGetLastError();
}

// Chunks per (sequence, kv head): at most one workgroup per CU (256 of them), each chunk a
// multiple of 128 tokens (one tile per wave at least).  A workgroup count a little above a
// multiple of the CU count gives a few CUs a second chunk while the rest idle, so the split
// rounds down; two per CU cost more merges and shorter per-wave streams.
void kv_split(int64_t batch, int64_t hkv, int64_t cap, int32_t *nsplit, int32_t *chunk)
{
    const int64_t want = 256 / (batch * hkv);
    const int64_t maxs = (cap + 127) / 128;
    int64_t ns = want < 1 ? 1 : (want > maxs ? maxs : want);
    if (ns > kKvMaxSplit) ns = kKvMaxSplit;
    int64_t ch = ((cap + ns - 1) / ns + 127) / 128 * 128;
    ns = (cap + ch - 1) / ch;
    *nsplit = (int32_t)ns;
    *chunk = (int32_t)ch;
}

}  // namespace qp
