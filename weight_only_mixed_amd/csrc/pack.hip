// Packing of unpacked codes into the page units and the device tile order.
//
// Units (mixed-bit page, s3.1): the smallest n with n*b divisible by 8 -- 4 values in 1
// byte (2-bit), 8 in 3 bytes (3-bit), 2 in 1 byte (4-bit), 8 in 5 bytes (5-bit), 4 in 3
// bytes (6-bit).  Value i of a unit occupies bits [b*i, b*i+b) of the little-endian integer
// formed by the unit's bytes (the shift sequences of s3.2).  Every 8 consecutive k of a row
// therefore form b whole bytes ("a block") whose little-endian value is sum_i q_i << (b*i).
// The canonical layout stores blocks in row order.  The device layout (a one-time repack,
// single-GPU 70B page, s3; documented in qpack.h) first reorders the values inside packing
// groups -- position p < G/2 holds value 2p, position G/2 + p value 2p + 1, with groups of 4
// k (6-bit), 8 k (3/4/5-bit) or the two 8-k blocks at k0 and k0 + 32, k0 % 64 < 32 (2-bit) --
// then packs each block the same way and moves its bytes to the tile order.  One thread
// handles one block (a 2-bit thread also reads its partner block's codes).
#include "qp_internal.h"

namespace qp {

// Byte offset of chunk byte c (0 <= c < 8*b) of lane `lane` inside a tile.
template <int B>
__device__ __forceinline__ int64_t dev_chunk_offset(int c, int lane)
{
    constexpr int F = 16 * (B / 2);
    return c < F ? (int64_t)(1024 * (c / 16) + 16 * lane + c % 16)
                 : (int64_t)(64 * F + 8 * lane + (c - F));
}

// Device offset of byte `i` of the block of row n starting at k0.
template <int B>
__device__ __forceinline__ int64_t dev_offset(int64_t n, int64_t k0, int i, int64_t k)
{
    const int64_t rb = n / kTileN, kt = k0 / kTileK;
    const int r = (int)(n % kTileN), kk = (int)(k0 % kTileK);
    const int gi = kk / 128, kq = kk % 128;
    const int j = 4 * gi + kq / 32, t = (kq % 32) / 8;
    const int lane = 16 * t + r;
    const int64_t tile = rb * (k / kTileK) + kt;
    return tile * 512 * B + dev_chunk_offset<B>(B * j + i, lane);
}

// Group value held at packed position p of a group of G values.
__device__ __forceinline__ int group_value(int G, int p) { return p < G / 2 ? 2 * p : 2 * (p - G / 2) + 1; }
// Packed position of group value v.
__device__ __forceinline__ int group_pos(int G, int v) { return (v & 1) ? G / 2 + v / 2 : v / 2; }

__device__ __forceinline__ uint64_t load8(const uint8_t *p) { return *(const uint64_t *)p; }

template <int B, int LAYOUT>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *codes, int64_t n, int64_t k,
                                                   uint8_t *out)
{
    const int64_t bpr = k / 8;
    const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx >= n * bpr) return;
    const int64_t row = idx / bpr, kb = idx % bpr, k0 = kb * 8;
    const uint8_t *crow = codes + row * k;
    uint64_t c8 = load8(crow + k0);  // the block's codes, value i in byte i
    if (LAYOUT == QP_LAYOUT_DEVICE) {
        uint8_t u[16];
        int h = 0;
        if (B == 2) {
            h = (k0 % 64) >= 32;  // second block of its group
            const int64_t ks = k0 - 32 * h;
            const uint64_t a = load8(crow + ks), b = load8(crow + ks + 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u[i] = (uint8_t)(a >> (8 * i));
                u[8 + i] = (uint8_t)(b >> (8 * i));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = (uint8_t)(c8 >> (8 * i));
        }
        uint64_t r = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            int v;
            if (B == 2) v = group_value(16, 8 * h + q);
            else if (B == 6) v = 4 * (q / 4) + group_value(4, q % 4);
            else v = group_value(8, q);
            r |= (uint64_t)u[v] << (8 * q);
        }
        c8 = r;
    }
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v |= ((c8 >> (8 * i)) & ((1u << B) - 1)) << (B * i);
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const int64_t off = LAYOUT == QP_LAYOUT_CANONICAL ? row * (k * B / 8) + kb * B + i
                                                          : dev_offset<B>(row, k0, i, k);
        out[off] = (uint8_t)(v >> (8 * i));
    }
}

// Codes of the block of `row` at k0, in packed position order (the bytes of the block read
// back through the layout's byte map).
template <int B, int LAYOUT>
__device__ __forceinline__ uint64_t read_block(const uint8_t *in, int64_t row, int64_t k0, int64_t k)
{
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const int64_t off = LAYOUT == QP_LAYOUT_CANONICAL ? row * (k * B / 8) + (k0 / 8) * B + i
                                                          : dev_offset<B>(row, k0, i, k);
        v |= (uint64_t)in[off] << (8 * i);
    }
    uint64_t c8 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) c8 |= ((v >> (B * i)) & ((1u << B) - 1)) << (8 * i);
    return c8;
}

template <int B, int LAYOUT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *in, int64_t n, int64_t k,
                                                     uint8_t *codes)
{
    const int64_t bpr = k / 8;
    const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (idx >= n * bpr) return;
    const int64_t row = idx / bpr, kb = idx % bpr, k0 = kb * 8;
    uint64_t c8 = read_block<B, LAYOUT>(in, row, k0, k);
    if (LAYOUT == QP_LAYOUT_DEVICE) {
        uint64_t other = 0;
        int h = 0;
        if (B == 2) {
            h = (k0 % 64) >= 32;
            other = read_block<B, LAYOUT>(in, row, h ? k0 - 32 : k0 + 32, k);
        }
        uint64_t r = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint64_t val;
            if (B == 2) {
                const int p = group_pos(16, 8 * h + i);  // position inside the 16-value group
                val = ((p / 8 == h ? c8 : other) >> (8 * (p % 8))) & 0xFF;
            } else if (B == 6) {
                val = (c8 >> (8 * (4 * (i / 4) + group_pos(4, i % 4)))) & 0xFF;
            } else {
                val = (c8 >> (8 * group_pos(8, i))) & 0xFF;
            }
            r |= val << (8 * i);
        }
        c8 = r;
    }
    *(uint64_t *)(codes + row * k + k0) = c8;
}

template <int B>
static hipError_t pack_bits(int layout, bool unpack, const uint8_t *src, int64_t n, int64_t k,
                            uint8_t *dst, hipStream_t st)
{
    const int64_t blocks = n * (k / 8);
    const dim3 grid((unsigned)((blocks + 255) / 256)), block(256);
    if (!unpack) {
        if (layout == QP_LAYOUT_CANONICAL)
            hipLaunchKernelGGL((pack_kernel<B, QP_LAYOUT_CANONICAL>), grid, block, 0, st, src, n, k, dst);
        else
            hipLaunchKernelGGL((pack_kernel<B, QP_LAYOUT_DEVICE>), grid, block, 0, st, src, n, k, dst);
    } else {
        if (layout == QP_LAYOUT_CANONICAL)
            hipLaunchKernelGGL((unpack_kernel<B, QP_LAYOUT_CANONICAL>), grid, block, 0, st, src, n, k, dst);
        else
            hipLaunchKernelGGL((unpack_kernel<B, QP_LAYOUT_DEVICE>), grid, block, 0, st, src, n, k, dst);
    }
    return hipGetLastError();
}

static hipError_t dispatch(int bits, int layout, bool unpack, const uint8_t *src, int64_t n,
                           int64_t k, uint8_t *dst, hipStream_t st)
{
    switch (bits) {
    case 2: return pack_bits<2>(layout, unpack, src, n, k, dst, st);
    case 3: return pack_bits<3>(layout, unpack, src, n, k, dst, st);
    case 4: return pack_bits<4>(layout, unpack, src, n, k, dst, st);
    case 5: return pack_bits<5>(layout, unpack, src, n, k, dst, st);
    case 6: return pack_bits<6>(layout, unpack, src, n, k, dst, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_pack(int bits, int layout, const uint8_t *codes, int64_t n, int64_t k,
                       uint8_t *out, hipStream_t st)
{
    return dispatch(bits, layout, false, codes, n, k, out, st);
}

hipError_t launch_unpack(int bits, int layout, const uint8_t *in, int64_t n, int64_t k,
                         uint8_t *codes, hipStream_t st)
{
    return dispatch(bits, layout, true, in, n, k, codes, st);
}

// Zero points in b bits (mixed-bit page, s2.3): one thread per 32-bit word of a row's
// little-endian stream, gathering the (at most 17) fields that overlap the word; group g's
// field is bits [g*b, g*b + b) of the row, bits past the last field are zero.
__global__ __launch_bounds__(256) void pack_zeros_kernel(const uint8_t *zeros, int64_t n, int64_t G, int bits,
                                                         int64_t words, uint32_t *out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * words) return;
    const int64_t r = i / words, w = i % words;
    const int64_t lo = 32 * w, hi = lo + 32;  // this word's bit range in the row stream
    uint32_t v = 0;
    for (int64_t g = lo / bits; g < G && g * bits < hi; ++g) {
        const uint64_t f = (uint64_t)(zeros[r * G + g] & ((1u << bits) - 1));
        const int64_t p = g * bits - lo;  // field position relative to the word (may be < 0)
        v |= (uint32_t)(p >= 0 ? f << p : f >> -p);
    }
    out[i] = v;
}

hipError_t launch_pack_zeros(int bits, const uint8_t *zeros, int64_t n, int64_t G, int64_t row_bytes,
                             uint8_t *out, hipStream_t st)
{
    const int64_t words = row_bytes / 4, total = n * words;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_zeros_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, zeros, n, G, bits,
                       words, (uint32_t *)out);
    return hipGetLastError();
}

}  // namespace qp
