// Raw buffer loads shared by the matmul kernels.
//
// A buffer resource covers [base, base + bytes); a load whose per-lane offset (voffset) is at
// or beyond `bytes` returns zeros instead of touching memory.  Wave-uniform parts of an
// address go in soffset (a scalar register), which keeps the per-lane address registers few.
// Every caller keeps soffset inside the range its voffset was checked against, so a load is
// in bounds whether or not the hardware includes soffset in the range check.
#pragma once

#include "qp_internal.h"

namespace qp {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ u4 ld16(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ u2 ld8(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t ld2(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}

// Wave-uniform value in a scalar register (for soffset).
__device__ __forceinline__ uint32_t uni(int64_t v) { return __builtin_amdgcn_readfirstlane((uint32_t)v); }

__device__ __forceinline__ float lo_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF)); }
__device__ __forceinline__ float hi_h(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }
__device__ __forceinline__ float h_f(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); }
// By value on purpose: __builtin_bit_cast applied directly to a vector element (v[i]) reads
// element 0 with this compiler.
__device__ __forceinline__ float as_f(uint32_t v) { return __builtin_bit_cast(float, v); }

// Two floats rounded to fp16 (nearest even) in one 32-bit word, first in the low half.
__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

}  // namespace qp
