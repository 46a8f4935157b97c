// Register-level unpack of the device layout into fp16 matrix-core operands.
//
// One lane of a wave holds, per 16-row x 256-k tile, a chunk of eight 8-k blocks of one
// weight row (b bytes each).  Block j feeds matrix-core step j as the lane's eight A-operand
// values, in k order.  A value (q - zp) is produced in fp16 exactly with the exponent-bias
// trick: OR-ing a code that sits at bit offset p (p + b <= 10) of a 16-bit half into the
// pattern of 1024.0 gives 1024 + 2^p*q exactly, and one packed fma
// (x * 2^-p - 1024*2^-p - zp) leaves q - zp, an exact small integer.  The device layout
// orders the values inside each packing group so that the two values of every pair
// (2i, 2i+1) of a block sit G/2*b bits apart in the chunk (16, 12, 16, 20, 12 bits for
// b = 2..6); one 32-bit window of the chunk then puts value 2i in the low half and value
// 2i+1 in the high half, each at an offset the bias trick accepts, and the pair costs one
// window (shift or v_alignbit_b32, shared where possible), one and-or and one packed fma.
// The per-group scale is applied later in fp32 (the mixed-bit page, s4.2, requires the
// scale multiply and the accumulation in fp32).
#pragma once

#include "qp_internal.h"

namespace qp {

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

// fp16 bits of -(1024*2^-p + zp) for a zero point zp < 2^(10-p): 1024*2^-p + zp has exponent
// 10 - p and mantissa zp*2^p, so the value is the sign and exponent bits of -1024*2^-p with
// zp*2^p in the mantissa.  The packed (lo, hi) pair for offsets (plo, phi) is therefore one
// integer multiply-add, zp * (2^plo + 2^(16+phi)) + bits(-1024*2^-plo, -1024*2^-phi), instead
// of two fp32 subtractions and a conversion.
__host__ __device__ constexpr uint32_t neg_bias_bits(int p) { return 0x8000u | ((uint32_t)(25 - p) << 10); }

template <int plo, int phi>
__device__ __forceinline__ h2 mul_const()
{
    h2 m;
    m[0] = (_Float16)(1.0f / (float)(1 << plo));
    m[1] = (_Float16)(1.0f / (float)(1 << phi));
    return m;
}

// 32 bits of a lane chunk d[0..NDW) starting at chunk bit ABS (ABS may be negative: the
// missing low bits are zeros; bits past the chunk end are zeros).
template <int ABS, int NDW>
__device__ __forceinline__ uint32_t window(const uint32_t *d)
{
    if constexpr (ABS < 0) {
        return d[0] << (-ABS);
    } else {
        constexpr int w = ABS / 32, o = ABS % 32;
        if constexpr (o == 0)
            return d[w];
        else if constexpr (w + 1 < NDW)
            return __builtin_amdgcn_alignbit(d[w + 1], d[w], o);
        else
            return d[w] >> o;
    }
}

// Where pair i (values 2i, 2i+1) of block J lives: the window start ABS (chunk bit), the
// value offsets PLO (low half) and PHI (high half) inside the window, and the index of the
// group constant (one per distinct offset pair).
template <int B, int J, int I> struct PairRule;
template <int J, int I> struct PairRule<2, J, I> {   // lo at 32*(J/2) + 8*(J%2) + 2I, gap 16
    static constexpr int ABS = 32 * (J / 2) + 8 * (J % 2), PLO = 2 * I, PHI = 2 * I, C = I;
};
template <int J, int I> struct PairRule<3, J, I> {   // lo at 24J + 3I, gap 12
    static constexpr int ABS = 24 * J + 3 * I - 4, PLO = 4, PHI = 0, C = 0;
};
template <int J, int I> struct PairRule<4, J, I> {   // lo at 32J + 4I, gap 16
    static constexpr int ABS = 32 * J + 8 * (I / 2), PLO = 4 * (I % 2), PHI = 4 * (I % 2), C = I % 2;
};
template <int J, int I> struct PairRule<5, J, I> {   // lo at 40J + 5I, gap 20
    static constexpr int ABS = 40 * J + 5 * I, PLO = 0, PHI = 4, C = 0;
};
template <int J, int I> struct PairRule<6, J, I> {   // lo at 48J + 24(I/2) + 6(I%2), gap 12
    static constexpr int ABS = 48 * J + 24 * (I / 2) + 6 * (I % 2) - 4, PLO = 4, PHI = 0, C = 0;
};

// Number of distinct (PLO, PHI) pairs per bit width, and pair c's offsets.
template <int B> struct Offsets;
template <> struct Offsets<2> { static constexpr int n = 4; static constexpr int plo[4] = {0, 2, 4, 6}; static constexpr int phi[4] = {0, 2, 4, 6}; };
template <> struct Offsets<3> { static constexpr int n = 1; static constexpr int plo[1] = {4}; static constexpr int phi[1] = {0}; };
template <> struct Offsets<4> { static constexpr int n = 2; static constexpr int plo[2] = {0, 4}; static constexpr int phi[2] = {0, 4}; };
template <> struct Offsets<5> { static constexpr int n = 1; static constexpr int plo[1] = {0}; static constexpr int phi[1] = {4}; };
template <> struct Offsets<6> { static constexpr int n = 1; static constexpr int plo[1] = {4}; static constexpr int phi[1] = {0}; };

// Per-group constants of the bias trick: add[c] = (-1024*2^-plo - zp, -1024*2^-phi - zp) for
// offset pair c, zp in [0, 2^B) (so zp < 2^(10-p) for every offset p with p + B <= 10).
template <int B> struct GroupConst {
    h2 add[Offsets<B>::n];
    __device__ __forceinline__ void set(uint32_t zp)
    {
#pragma unroll
        for (int i = 0; i < Offsets<B>::n; ++i) {
            const uint32_t c = neg_bias_bits(Offsets<B>::plo[i]) | (neg_bias_bits(Offsets<B>::phi[i]) << 16);
            const uint32_t mult = (1u << Offsets<B>::plo[i]) | (1u << (16 + Offsets<B>::phi[i]));
            add[i] = bits_h2((zp & ((1u << B) - 1)) * mult + c);
        }
    }
};

template <int B, int J, int I>
__device__ __forceinline__ uint32_t unpack_pair(const uint32_t *d, const GroupConst<B> &gc)
{
    using R = PairRule<B, J, I>;
    static_assert(R::PLO + B <= 10 && R::PHI + B <= 10, "field must stay inside the fp16 mantissa");
    static_assert(Offsets<B>::plo[R::C] == R::PLO && Offsets<B>::phi[R::C] == R::PHI, "offset table");
    constexpr uint32_t mask = (((1u << B) - 1) << R::PLO) | (((1u << B) - 1) << (16 + R::PHI));
    return magic_pair<mask>(window<R::ABS, 2 * B>(d), mul_const<R::PLO, R::PHI>(), gc.add[R::C]);
}

// Unpack block J (0..7) of a lane chunk d[2*B] into 8 fp16 values (q - zp), k order.
template <int B, int J> struct BlockUnpack {
    static __device__ __forceinline__ h8 run(const uint32_t *d, const GroupConst<B> &gc)
    {
        u4 r;
        r[0] = unpack_pair<B, J, 0>(d, gc);
        r[1] = unpack_pair<B, J, 1>(d, gc);
        r[2] = unpack_pair<B, J, 2>(d, gc);
        r[3] = unpack_pair<B, J, 3>(d, gc);
        return __builtin_bit_cast(h8, r);
    }
};

// Unpack all eight blocks of a chunk with NG groups per k-tile: block j belongs to group
// j * NG / 8 (NG = 2: blocks 0-3 and 4-7; NG = 8: one group per block).
template <int B, int NG>
__device__ __forceinline__ void unpack_chunk_groups(const uint32_t *d, const GroupConst<B> (&gc)[NG], h8 *a)
{
    a[0] = BlockUnpack<B, 0>::run(d, gc[0 * NG / 8]);
    a[1] = BlockUnpack<B, 1>::run(d, gc[1 * NG / 8]);
    a[2] = BlockUnpack<B, 2>::run(d, gc[2 * NG / 8]);
    a[3] = BlockUnpack<B, 3>::run(d, gc[3 * NG / 8]);
    a[4] = BlockUnpack<B, 4>::run(d, gc[4 * NG / 8]);
    a[5] = BlockUnpack<B, 5>::run(d, gc[5 * NG / 8]);
    a[6] = BlockUnpack<B, 6>::run(d, gc[6 * NG / 8]);
    a[7] = BlockUnpack<B, 7>::run(d, gc[7 * NG / 8]);
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace qp
