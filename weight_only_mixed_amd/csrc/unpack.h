// Register-level unpack of the device layout into fp16 matrix-core operands.
//
// One lane of a wave holds, per 16-row x 256-k tile, a chunk of eight 8-k blocks of one
// weight row (b bytes each; the canonical page units kept whole).  Block j feeds matrix-core
// step j as the lane's eight A-operand values, in k order.  A value (q - zp) is produced in
// fp16 exactly with the exponent-bias trick: OR-ing a code that sits at bit offset p < 10 of
// a 16-bit half into the pattern of 1024.0 gives 1024 + 2^p*q exactly, and one packed fma
// (x * 2^-p - 1024*2^-p - zp) leaves q - zp, an exact small integer.  Both halves of a
// 32-bit word are converted by one and-or plus one packed fma; each half has its own offset.
// The per-group scale is applied later in fp32 (the mixed-bit page, s4.2, requires the
// scale multiply and the accumulation in fp32).
#pragma once

#include "qp_internal.h"

namespace qp {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Bits [A, A+32) of the 64-bit value {hi, lo} (zeros above bit 63), A compile-time.
// Written with v_alignbit_b32 rather than 64-bit shifts: the compiler may fuse a 64-bit
// shift of two adjacent array elements into one 64-bit access, which keeps the register
// array from being split into registers.
template <int A>
__device__ __forceinline__ uint32_t win(uint32_t hi, uint32_t lo)
{
    static_assert(A >= 0 && A < 64, "window offset");
    if constexpr (A == 0)
        return lo;
    else if constexpr (A < 32)
        return __builtin_amdgcn_alignbit(hi, lo, A);
    else if constexpr (A == 32)
        return hi;
    else
        return hi >> (A - 32);
}

__device__ __forceinline__ uint32_t bfi_hi(uint32_t hi_src, uint32_t lo_src)
{
    return (hi_src & 0xFFFF0000u) | (lo_src & 0x0000FFFFu);
}

__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 bits_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// A constant the compiler keeps in a vector register.  (word & mask) | bias is then one
// v_and_or_b32 (the bias sits in a scalar register); with both constants as literals the
// compiler emits a separate and and or.  The empty non-volatile asm is hoisted out of loops.
template <uint32_t M>
__device__ __forceinline__ uint32_t vconst()
{
    uint32_t v = M;
    asm("" : "+v"(v));
    return v;
}

// (word & MASK) | bias(1024.0 in both halves), then * mul + add, in packed fp16.
template <uint32_t MASK>
__device__ __forceinline__ uint32_t magic_pair(uint32_t word, h2 mul, h2 add)
{
    const uint32_t t = (word & vconst<MASK>()) | 0x64006400u;
    return h2_bits(__builtin_elementwise_fma(bits_h2(t), mul, add));
}

// Packed (lo, hi) constants -1024*2^-p - zp for one group's zero point.
__device__ __forceinline__ h2 add_const(float clo, float chi, float zp)
{
    return __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(clo - zp, chi - zp));
}

// Per-bitwidth pair offsets.  For each pair v (values 2v, 2v+1 of a block) the low half
// carries value 2v at offset PLO and the high half value 2v+1 at offset PHI.
template <int B> struct Offsets;
template <> struct Offsets<2> { static constexpr int n = 2; static constexpr int plo[2] = {0, 4}; static constexpr int phi[2] = {2, 6}; };
template <> struct Offsets<3> { static constexpr int n = 2; static constexpr int plo[2] = {0, 6}; static constexpr int phi[2] = {0, 6}; };
template <> struct Offsets<4> { static constexpr int n = 1; static constexpr int plo[1] = {0}; static constexpr int phi[1] = {4}; };
template <> struct Offsets<5> { static constexpr int n = 1; static constexpr int plo[1] = {0}; static constexpr int phi[1] = {5}; };
template <> struct Offsets<6> { static constexpr int n = 1; static constexpr int plo[1] = {0}; static constexpr int phi[1] = {0}; };

template <int B> struct GroupConst {
    h2 add[Offsets<B>::n];
    __device__ __forceinline__ void set(uint32_t zp)
    {
        float z = (float)zp;
#pragma unroll
        for (int i = 0; i < Offsets<B>::n; ++i)
            add[i] = add_const(-1024.0f / (float)(1 << Offsets<B>::plo[i]),
                               -1024.0f / (float)(1 << Offsets<B>::phi[i]), z);
    }
};

template <int plo, int phi>
__device__ __forceinline__ h2 mul_const()
{
    h2 m;
    m[0] = (_Float16)(1.0f / (float)(1 << plo));
    m[1] = (_Float16)(1.0f / (float)(1 << phi));
    return m;
}

// Unpack block J (0..7) of a lane chunk d[2*B] into 8 fp16 values (q - zp), k order.
template <int B, int J> struct BlockUnpack;

// 2-bit: block = bytes 2J, 2J+1 (dword J/2); value i at bit 2i of the 16-bit block.
template <int J> struct BlockUnpack<2, J> {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<2> &gc)
    {
        const uint32_t D = d[J / 2];
        constexpr uint32_t b0 = 2 * (J % 2), b1 = b0 + 1;
        const uint32_t xa = perm(D, D, b0 | (b1 << 8) | (b0 << 16) | (b1 << 24));
        const uint32_t xb = perm(D, D, b1 | (b1 << 8) | (b1 << 16) | (b1 << 24));
        u4 r;
        r[0] = magic_pair<0x000C0003u>(xa, mul_const<0, 2>(), gc.add[0]);
        r[1] = magic_pair<0x00C00030u>(xa, mul_const<4, 6>(), gc.add[1]);
        r[2] = magic_pair<0x000C0003u>(xb, mul_const<0, 2>(), gc.add[0]);
        r[3] = magic_pair<0x00C00030u>(xb, mul_const<4, 6>(), gc.add[1]);
        return __builtin_bit_cast(h8, r);
    }
};

// 3-bit: block = one 3-byte unit at chunk byte 3J; value i at bit 3i.
template <int J> struct BlockUnpack<3, J> {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<3> &gc)
    {
        constexpr int c = 3 * J, w = c / 4, s = 8 * (c % 4);
        uint32_t v;
        if constexpr ((c % 4) + 3 <= 4)
            v = d[w] >> s;                 // unit inside one dword
        else
            v = win<s>(d[w + 1], d[w]);    // unit straddles two dwords
        const uint32_t w1 = bfi_hi(v << 13, v);          // lo: v[0:16)  hi: v[3:19)
        const uint32_t w2 = bfi_hi(v << 1, v >> 12);     // lo: v[12:28) hi: v[15:31)
        u4 r;
        r[0] = magic_pair<0x00070007u>(w1, mul_const<0, 0>(), gc.add[0]);
        r[1] = magic_pair<0x01C001C0u>(w1, mul_const<6, 6>(), gc.add[1]);
        r[2] = magic_pair<0x00070007u>(w2, mul_const<0, 0>(), gc.add[0]);
        r[3] = magic_pair<0x01C001C0u>(w2, mul_const<6, 6>(), gc.add[1]);
        return __builtin_bit_cast(h8, r);
    }
};

// 4-bit: block = dword J; value i at bit 4i (low nibble first).
template <int J> struct BlockUnpack<4, J> {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<4> &gc)
    {
        const uint32_t D = d[J];
        u4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = perm(D, D, (uint32_t)i * 0x01010101u);
            r[i] = magic_pair<0x00F0000Fu>(x, mul_const<0, 4>(), gc.add[0]);
        }
        return __builtin_bit_cast(h8, r);
    }
};

// 5-bit: block = one 5-byte unit at chunk byte 5J; value i at bit 5i of 40 bits.
template <int J> struct BlockUnpack<5, J> {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<5> &gc)
    {
        constexpr int c = 5 * J, w = c / 4, o = c % 4, s = 8 * o;
        const uint32_t lo = d[w], hi = d[w + 1];
        constexpr uint32_t sel = o | ((o + 1) << 8) | (o << 16) | ((o + 1) << 24);
        const uint32_t x0 = perm(hi, lo, sel);           // both halves: v[0:16)
        const uint32_t a1 = win<s + 10>(hi, lo), a2 = win<s + 20>(hi, lo), a3 = win<s + 30>(hi, lo);
        const uint32_t x1 = perm(a1, a1, 0x01000100u);
        const uint32_t x2 = perm(a2, a2, 0x01000100u);
        const uint32_t x3 = perm(a3, a3, 0x01000100u);
        u4 r;
        r[0] = magic_pair<0x03E0001Fu>(x0, mul_const<0, 5>(), gc.add[0]);
        r[1] = magic_pair<0x03E0001Fu>(x1, mul_const<0, 5>(), gc.add[0]);
        r[2] = magic_pair<0x03E0001Fu>(x2, mul_const<0, 5>(), gc.add[0]);
        r[3] = magic_pair<0x03E0001Fu>(x3, mul_const<0, 5>(), gc.add[0]);
        return __builtin_bit_cast(h8, r);
    }
};

// 6-bit: block = two 3-byte units at chunk byte 6J; value i at bit 6i of 48 bits.
template <int J> struct BlockUnpack<6, J> {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<6> &gc)
    {
        constexpr int c = 6 * J, w = c / 4, s = 8 * (c % 4);
        const uint32_t lo = d[w], hi = d[w + 1];
        const uint32_t v0 = win<s>(hi, lo);
        const uint32_t w0 = bfi_hi(v0 << 10, v0);                                  // q0, q1
        const uint32_t w1 = bfi_hi(win<s + 2>(hi, lo), win<s + 12>(hi, lo));        // q2, q3
        const uint32_t w2 = bfi_hi(win<s + 14>(hi, lo), win<s + 24>(hi, lo));       // q4, q5
        const uint32_t w3 = bfi_hi(win<s + 26>(hi, lo), win<s + 36>(hi, lo));       // q6, q7
        u4 r;
        r[0] = magic_pair<0x003F003Fu>(w0, mul_const<0, 0>(), gc.add[0]);
        r[1] = magic_pair<0x003F003Fu>(w1, mul_const<0, 0>(), gc.add[0]);
        r[2] = magic_pair<0x003F003Fu>(w2, mul_const<0, 0>(), gc.add[0]);
        r[3] = magic_pair<0x003F003Fu>(w3, mul_const<0, 0>(), gc.add[0]);
        return __builtin_bit_cast(h8, r);
    }
};

// Load lane `lane`'s chunk of one device-layout tile (512*B bytes at `tile`).
template <int B>
__device__ __forceinline__ void load_chunk(const uint8_t *tile, int lane, uint32_t *d)
{
#pragma unroll
    for (int s = 0; s < B / 2; ++s) {
        const u4 v = *(const u4 *)(tile + 1024 * s + 16 * lane);
        d[4 * s + 0] = v[0];
        d[4 * s + 1] = v[1];
        d[4 * s + 2] = v[2];
        d[4 * s + 3] = v[3];
    }
    if (B & 1) {
        const u2 v = *(const u2 *)(tile + 1024 * (B / 2) + 8 * lane);
        d[2 * B - 2] = v[0];
        d[2 * B - 1] = v[1];
    }
}

// Unpack all eight blocks of a chunk; blocks 0..3 use group 0's zero point, 4..7 group 1's.
template <int B>
__device__ __forceinline__ void unpack_chunk(const uint32_t *d, const GroupConst<B> &g0,
                                             const GroupConst<B> &g1, h8 *a)
{
    a[0] = BlockUnpack<B, 0>::run(d, g0);
    a[1] = BlockUnpack<B, 1>::run(d, g0);
    a[2] = BlockUnpack<B, 2>::run(d, g0);
    a[3] = BlockUnpack<B, 3>::run(d, g0);
    a[4] = BlockUnpack<B, 4>::run(d, g1);
    a[5] = BlockUnpack<B, 5>::run(d, g1);
    a[6] = BlockUnpack<B, 6>::run(d, g1);
    a[7] = BlockUnpack<B, 7>::run(d, g1);
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// First k of block j of lane group t inside k-tile kt.
__device__ __forceinline__ int block_k0(int kt, int j, int t)
{
    return kTileK * kt + 128 * (j >> 2) + 32 * (j & 3) + 8 * t;
}

}  // namespace qp
