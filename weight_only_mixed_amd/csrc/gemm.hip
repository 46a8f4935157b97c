// Prefill dequant-GEMM: the outlier add-back kernels and the dispatch over bit width, group
// size and zero-point form (the matrix-core kernel itself is in gemm_kernel.h).  Groups of 128
// with byte or implied zero points are instantiated here.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(128, kZpByte)
QP_GEMM_VARIANT_EXTERN(64, kZpByte)
QP_GEMM_VARIANT_EXTERN(32, kZpByte)
QP_GEMM_VARIANT_EXTERN(128, kZpPacked)
QP_GEMM_VARIANT_EXTERN(64, kZpPacked)
QP_GEMM_VARIANT_EXTERN(32, kZpPacked)
QP_GEMM_VARIANT_EXTERN(128, kZpFp8)
QP_GEMM_VARIANT_EXTERN(64, kZpFp8)
QP_GEMM_VARIANT_EXTERN(32, kZpFp8)
}  // namespace gk

// Position of activation row 16 mt + 4 t + i (of a 128-row block) in the transposed layouts:
// 32 t + 4 mt + i, so a GEMM lane (t, r) finds its eight tiles' rows as 32 consecutive values.
__device__ __forceinline__ int xt_row(int p) { return 16 * ((p & 31) >> 2) + 4 * (p >> 5) + (p & 3); }

// x^T for the outlier partial: xt[kk][128 mb + p] = x[128 mb + xt_row(p)][kk], zeros for rows
// >= m.  One block per 64 k x 128 m tile: 16-byte loads of x rows into LDS, then each thread
// gathers eight positions for one 16-byte store of x^T.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                                                        uint16_t *xt, int64_t ldxt)
{
    constexpr int kPitch = 64 + 2;  // halves per LDS row (odd dword pitch: rows hit distinct banks)
    __shared__ uint16_t tile[128 * kPitch];
    const int64_t k0 = blockIdx.x * 64, m0 = blockIdx.y * 128;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + 256 * it, row = idx / 8, c = idx % 8;
        const int64_t gm = m0 + row, gk = k0 + 8 * c;
        u4 v = {0u, 0u, 0u, 0u};
        if (gm < m && gk < k) v = *(const u4 *)(x + gm * ldx + gk);
        uint32_t *dst = (uint32_t *)(tile + row * kPitch + 8 * c);  // 4-byte aligned: kPitch even
        dst[0] = v[0];
        dst[1] = v[1];
        dst[2] = v[2];
        dst[3] = v[3];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = threadIdx.x + 256 * it, kk = idx / 16, sgm = idx % 16;  // positions 8 sgm ..
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            w[h] = (uint32_t)tile[xt_row(8 * sgm + 2 * h) * kPitch + kk] |
                   ((uint32_t)tile[xt_row(8 * sgm + 2 * h + 1) * kPitch + kk] << 16);
        const int64_t gk = k0 + kk;
        if (gk < k) *(u4 *)(xt + gk * ldxt + m0 + 8 * sgm) = (u4){w[0], w[1], w[2], w[3]};
    }
}

// Outlier partial: S^T[n][p] = sum over the outliers (n, c, v) of v * x^T[c][p], in fp32.  A
// wave takes eight weight rows and one 64-position chunk: lane (8 j + q) sums row 8 w + j over
// positions 8 q .. 8 q + 7 of the chunk.  Per step the eight lanes of a row load sixteen of its
// entries (two each) and pass them round, so all sixteen 16-byte gathers are in flight behind
// one index load.  Work items (chunk, 32-row group) run chunk-major and each XCD (workgroup b on
// XCD b % 8) takes a contiguous eighth of them, so an XCD gathers from about one chunk of x^T at
// a time (k rows of 128 bytes: L2-resident) rather than from all of it.
__global__ __launch_bounds__(256) void outlier_spmm_kernel(const int32_t *rowptr, const int32_t *col,
                                                           const uint16_t *val, const uint16_t *xt, int64_t n,
                                                           int64_t k, int64_t ldxt, int64_t per_xcd, float *spart)
{
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int64_t groups = (n + 31) / 32, chunk = item / groups;
    if (chunk >= ldxt / 64) return;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane & 7;
    const int64_t row = (item % groups) * 32 + 8 * wv + (lane >> 3);
    if (row >= n) return;  // whole eight-lane row groups: the exchanges below stay inside one
    const int64_t p = chunk * 64 + 8 * q;
    const rsrc_t xr = make_rsrc(xt, k * ldxt * 2);  // (under 2 GiB) a column index outside k reads zeros
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t e0 = rowptr[row], e1 = rowptr[row + 1];
    for (int64_t e = e0; e < e1; e += 16) {
        int32_t c2[2];
        uint32_t v2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool ok = e + 8 * h + q < e1;
            c2[h] = ok ? col[e + 8 * h + q] : -1;
            v2[h] = ok ? val[e + 8 * h + q] : 0u;
        }
        u4 xv[16];
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int src = (lane & ~7) | (j & 7);
            const int32_t c = __shfl(c2[j >> 3], src);
            v[j] = h_f((uint16_t)__shfl((int)v2[j >> 3], src));
            xv[j] = ld16(xr, (uint64_t)c < (uint64_t)k ? (uint32_t)(((int64_t)c * ldxt + p) * 2) : 0x80000000u);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[2 * u] = __builtin_fmaf(lo_h(xv[j][u]), v[j], acc[2 * u]);
                acc[2 * u + 1] = __builtin_fmaf(hi_h(xv[j][u]), v[j], acc[2 * u + 1]);
            }
    }
    f4 *dst = (f4 *)(spart + row * ldxt + p);
    dst[0] = (f4){acc[0], acc[1], acc[2], acc[3]};
    dst[1] = (f4){acc[4], acc[5], acc[6], acc[7]};
}

int64_t gemm_xt_ld(int64_t m) { return (m + gk::GeoLayer::kMRows - 1) / gk::GeoLayer::kMRows * gk::GeoLayer::kMRows; }

// Split k when the output tiles fill at most half of the CUs: double the parts while the
// workgroups stay within one per CU and each part keeps whole 512-k tile pairs (at most 8).
int gemm_split_parts(int64_t m, int64_t n, int64_t k)
{
    constexpr int64_t kCUs = 256;
    const int64_t tiles = (n + gk::GeoLayer::kNT - 1) / gk::GeoLayer::kNT * ((m + gk::GeoLayer::kMRows - 1) / gk::GeoLayer::kMRows);
    int s = 1;
    while (s < 8 && tiles * 2 * s <= kCUs && k % (512 * 2 * s) == 0) s *= 2;
    return s;
}

// The split GEMM's reduction: y[r][c] = fp16(sum of the ksplit fp32 partials in part order),
// rounded once (the first part started from the outlier partial).  Four outputs per thread.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *parts, int32_t nparts, int64_t pstride,
                                                           int64_t m, int64_t n, uint16_t *y, int64_t ldy)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (row, 4-column) index
    const int64_t q = n / 4;
    if (i >= m * q) return;
    const int64_t row = i / q, c = 4 * (i % q);
    f4 acc = *(const f4 *)(parts + row * n + c);
    for (int32_t s = 1; s < nparts; ++s) acc += *(const f4 *)(parts + s * pstride + row * n + c);
    uint16_t *dst = y + row * ldy + c;
    *(u2 *)dst = (u2){pack_h2(acc[0], acc[1]), pack_h2(acc[2], acc[3])};
}

template <int ZPK>
static hipError_t gemm_zp(int bits, bool outl, const GemmArgs &a, hipStream_t st)
{
    switch (a.gs) {
    case 128: return gk::gemm_main<128, ZPK>(bits, outl, a, st);
    case 64: return gk::gemm_main<64, ZPK>(bits, outl, a, st);
    case 32: return gk::gemm_main<32, ZPK>(bits, outl, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(int bits, const GemmArgs &a, hipStream_t st)
{
    if (a.rowptr) {
        hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((a.k + 63) / 64), (unsigned)(a.ldxt / 128)), dim3(256), 0,
                           st, a.x, a.ldx, a.m, a.k, a.xt, a.ldxt);
        const int64_t per_xcd = ((a.n + 31) / 32 * (a.ldxt / 64) + 7) / 8;
        hipLaunchKernelGGL(outlier_spmm_kernel, dim3((unsigned)(8 * per_xcd)), dim3(256), 0, st, a.rowptr, a.col,
                           a.val, a.xt, a.n, a.k, a.ldxt, per_xcd, a.spart);
    }
    if (a.ksplit > 1) {
        // k parts into fp32 partial rows (the first seeded from the outlier partial), then one
        // pass sums them
        GemmArgs g = a;
        if (!a.rowptr) g.spart = nullptr;
        g.y = a.parts;
        g.ldy = a.n;
        g.ysplit = a.m * a.n;
        hipError_t e = a.fp8    ? gemm_zp<gk::kZpFp8>(bits, false, g, st)
                       : a.zrow ? gemm_zp<gk::kZpPacked>(bits, false, g, st)
                                : gemm_zp<gk::kZpByte>(bits, false, g, st);
        if (e != hipSuccess) return e;
        const int64_t items = a.m * (a.n / 4);
        hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a.parts,
                           a.ksplit, a.m * a.n, a.m, a.n, (uint16_t *)a.y, a.ldy);
        return hipGetLastError();
    }
    if (a.fp8) return gemm_zp<gk::kZpFp8>(bits, a.rowptr != nullptr, a, st);
    return a.zrow ? gemm_zp<gk::kZpPacked>(bits, a.rowptr != nullptr, a, st)
                  : gemm_zp<gk::kZpByte>(bits, a.rowptr != nullptr, a, st);
}

template <int ZPK>
static hipError_t grouped_zp(int bits, int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    switch (a.gs) {
    case 128: return gk::grouped_main<128, ZPK>(bits, epilogue, n_experts, a, st);
    case 64: return gk::grouped_main<64, ZPK>(bits, epilogue, n_experts, a, st);
    case 32: return gk::grouped_main<32, ZPK>(bits, epilogue, n_experts, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(int bits, int epilogue, int n_experts, const GemmArgs &a, hipStream_t st)
{
    if (a.m < 1) return hipSuccess;
    if (a.fp8) return grouped_zp<gk::kZpFp8>(bits, epilogue, n_experts, a, st);
    return a.zrow ? grouped_zp<gk::kZpPacked>(bits, epilogue, n_experts, a, st)
                  : grouped_zp<gk::kZpByte>(bits, epilogue, n_experts, a, st);
}

}  // namespace qp
