// Internal declarations shared by the HIP translation units of libqpack.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qpack.h"

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

namespace qp {

constexpr int kGroup = 128;      // weights per (scale, zero point)
constexpr int kTileN = 16;       // rows per device-layout tile
constexpr int kTileK = 256;      // k per device-layout tile (two groups)
constexpr int kMaxExperts = 64;  // experts per grouped launch (kernel-argument table)

// ---- host-side helpers (api.hip) ---------------------------------------------------
qp_status fail(qp_status st, const char *fmt, ...);
qp_status check_launch(const char *what);

// ---- launchers -----------------------------------------------------------------------
struct QuantWs {  // carve-up of the quantize workspace
    uint32_t *hist;      // [32768] magnitude histogram
    uint32_t *ctl;       // [4]: threshold bits, need_eq lo/hi, spare
    int32_t *gt_cnt;     // [n]
    int32_t *eq_cnt;     // [n]
    int32_t *eq_base;    // [n]
};
size_t quant_ws_bytes(int64_t n);
QuantWs quant_ws_carve(void *ws, int64_t n);
hipError_t launch_quantize(int bits, bool sym, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                           int64_t kout, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                           int32_t *rowptr, int32_t *col, uint16_t *val, const QuantWs &ws,
                           hipStream_t st);

hipError_t launch_pack(int bits, int layout, const uint8_t *codes, int64_t n, int64_t k,
                       uint8_t *out, hipStream_t st);
hipError_t launch_unpack(int bits, int layout, const uint8_t *in, int64_t n, int64_t k,
                         uint8_t *codes, hipStream_t st);
hipError_t launch_pack_zeros(int bits, const uint8_t *zeros, int64_t n, int64_t G, int64_t row_bytes,
                             uint8_t *out, hipStream_t st);

// One quantized weight's device buffers.  With fp8 scales, `scales` holds the E4M3 scale
// bytes [n][k/gs] (read as bytes), rowf the fp32 row factors [n] and fb the fp16 fallback
// scales [n][fb_stride] (null with fb_stride 0); with fp16 scales rowf and fb are null.
struct ExpertPtrs {
    const uint8_t *packed;
    const uint16_t *scales;
    const uint8_t *zeros;
    const float *rowf;
    const uint16_t *fb;
    int32_t fb_stride;
};
// One decode GEMV problem, and a batch of independent ones run in a single launch.
constexpr int kMaxGemvBatch = 8;
struct GemvProblem {
    ExpertPtrs w;
    const int32_t *rowptr;  // outlier CSR, or null
    const int32_t *col;
    const uint16_t *val;
    const uint16_t *x;
    int64_t ldx;
    int64_t m, n, k;
    uint16_t *y;
    int64_t ldy;
    int32_t bits;
    uint32_t zmid;   // 0: stored zero points; else the implied pair (2^(b-1) in both bytes)
    int32_t gs;      // group size: 32, 64 or 128
    int32_t zrow;    // bytes per row of b-bit zero points (0: one byte per group)
    int64_t block0;  // batch: first workgroup of this problem
    int32_t fp8;     // 1: E4M3 scales (w.scales holds the bytes, w.rowf and w.fb are set)
};
struct GemvBatch {
    GemvProblem p[kMaxGemvBatch];
    int32_t count;
};
hipError_t launch_gemv(const GemvProblem &p, hipStream_t st);
int64_t quantize_fp8_max_groups();
hipError_t launch_quantize_fp8(int bits, bool sym, const uint16_t *w, int64_t ldw, int64_t n, int64_t k, int gs,
                               uint8_t *codes, uint8_t *sc8, uint8_t *zeros, float *factors, uint16_t *fb,
                               int64_t fb_stride, int32_t *counts, hipStream_t st);
hipError_t launch_gemv_batch(const GemvBatch &b, int64_t blocks, int m_max, hipStream_t st);

// Dequant-GEMM on the matrix cores: a plain layer (ex[0], optional outliers) or a group of
// routed experts (ex[e] over the sorted rows offsets[e] .. offsets[e+1]).
struct GemmArgs {
    ExpertPtrs ex[kMaxExperts];
    const int32_t *rowptr;   // outlier CSR (plain layer only), or null
    const int32_t *col;
    const uint16_t *val;
    const uint16_t *x;
    int64_t ldx;
    const int32_t *row_src;  // grouped: row of x feeding sorted row r (null: row r)
    const int32_t *offsets;  // grouped: [n_experts + 1] sorted-row ranges
    int64_t m, n, k;         // grouped: m = upper bound of the sorted rows (and of x's rows)
    void *y;
    int64_t ldy;
    uint32_t zmid;  // 0: stored zero points; else the implied pair (2^(b-1) in both bytes)
    uint32_t zrow;  // 0: one zero-point byte per group; else bytes per row of b-bit zero points
    int32_t gs;     // group size: 128, 64 or 32
    int32_t ksplit;  // fp32 rows: k in ksplit equal parts (0 or 1: whole k); part s writes its
    int64_t ysplit;  //   partial rows at y + s * ysplit floats (grouped), or at parts + s * ysplit
                     //   (the layer GEMM, summed into y by the split reduction)
    float *parts;    // layer GEMM with ksplit > 1: workspace of ksplit fp32 [m][n] partials
    int32_t fp8;    // 1: E4M3 scales for every expert (ex[e].scales holds the bytes)
    uint16_t *xt;   // workspace (outliers only): x transposed, [k][ldxt]
    float *spart;   // workspace (outliers only): fp32 outlier partial, [n][ldxt]
    int64_t ldxt;
};
int64_t gemm_xt_ld(int64_t m);
// k parts the layer GEMM splits into for an m x n output with k columns (1: no split): enough
// to give the GPU's CUs a workgroup each when the output tiles alone leave most idle.
int gemm_split_parts(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm(int bits, const GemmArgs &a, hipStream_t st);
hipError_t launch_grouped(int bits, int epilogue, int n_experts, const GemmArgs &a, hipStream_t st);

// Integer-dot path: per-token int8 activations (storage map of qpack.h) and the GEMM on them.
hipError_t launch_act_quantize(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int8_t *xq, float *scales,
                               hipStream_t st);
hipError_t launch_gemm_a8(int bits, const ExpertPtrs &w, bool fp8, const int8_t *xq, const float *sx, int64_t m,
                          int64_t n, int64_t k, uint32_t zmid, uint32_t zrow, uint16_t *y, int64_t ldy, hipStream_t st);

hipError_t launch_moe_dispatch(const int32_t *ids, const float *w, int64_t tokens, int topk,
                               int n_experts, int32_t *offsets, int32_t *row_src,
                               float *row_weight, int32_t *token_rows, hipStream_t st);
hipError_t launch_moe_combine(const float *rows, int64_t ld_rows, const int32_t *token_rows,
                              const float *row_weight, int64_t tokens, int topk, int64_t n,
                              uint16_t *out, int64_t ldo, int nsplit, int64_t split_stride,
                              hipStream_t st);

}  // namespace qp
