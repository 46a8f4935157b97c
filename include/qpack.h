/*
 * qpack.h -- C ABI of the MI355X (gfx950) weight-only mixed-bit quantized linear layer.
 *
 * Weights W[n][k] (n = output feature, k = input feature) are quantized to b = 2..6 bits
 * with one fp16 scale and one integer zero point per group of g = 128 (or 64, 32)
 * consecutive k of a row, packed in the page units, dequantized on the GPU and multiplied by
 * fp16 activations:
 *     y[m][n] = sum_k x[m][k] * (q[n][k] - zp[n][k/g]) * s[n][k/g]
 *             + sum_{(n,k) in outliers} x[m][k] * w[n][k].
 *
 * Passages this interface follows (page title, section):
 *  - quantization formula scale=(max-min)/(qmax-qmin), zero_point=qmin-round(min/scale),
 *    q=round(x/scale)+zero_point, x_hat=(q-zero_point)*scale:
 *    "大模型推理加速实战：量化、投机采样与PD分离的工程指南", s1.1;
 *  - groups of 128, top-0.1% |w| held out in fp16 and added back after the GEMM, fused
 *    dequant-GEMM argument list (a, b, c, scale, zero_point, M, N, K, strides), unfused
 *    reference dequantize -> matmul(x, W^T), one-time device repack:
 *    "单卡运行70B大模型的五层技术栈实战", s2 and s3;
 *  - packing units (2-bit: 4 values/1 byte, 3-bit: 8/3, 5-bit: 8/5, 6-bit: 4/3), LSB-first
 *    values in little-endian units, fp16 scales, fp32 scale multiply, scales ordered to
 *    match GPU tiles: 2/3/5/6-bit mixed quantization page (pwwt.cn), s2.3, s3.1-s3.3, s4.2;
 *  - 4-bit packs two values per byte: KV-cache quantization page (kwkr.cn), s5.1;
 *  - routed experts receive hidden states plus top-k expert ids:
 *    "端侧MoE推理存储墙优化：显存精算、预取重叠与量化补偿实战", s4.2;
 *  - quantized KV cache read directly by decode attention: KV-cache quantization page
 *    (kwkr.cn), s2.1-s2.3, s3.1, s5.1.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers (hipMalloc'd memory, e.g. torch tensors), except
 *    where a parameter says "host".  The caller owns and allocates every buffer; the library
 *    allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls are
 *    asynchronous on that stream; no call synchronizes the device.
 *  - Arguments are validated on the host before anything is launched.  On any status other
 *    than QP_OK nothing has been written, except QP_ERR_DEVICE (a launch failed; outputs are
 *    undefined).  qp_last_error() then returns a message for the calling thread.
 *  - No C++ exception crosses this interface.  Inputs must be finite (not checked).
 *  - fp16 values are passed as their uint16_t bit patterns.
 */
#ifndef QPACK_H
#define QPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QP_OK = 0,
    QP_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment or stride */
    QP_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. group size other than 128) */
    QP_ERR_DEVICE = 3,      /* a HIP launch failed; message in qp_last_error() */
    QP_ERR_WORKSPACE = 4    /* workspace or CSR capacity too small */
} qp_status;

/* Packed-byte layouts.
 * QP_LAYOUT_CANONICAL: row n occupies k*bits/8 bytes; row n's codes in k order are cut into
 *   page units (u values per unit: 4, 8, 2, 8, 4 for b = 2, 3, 4, 5, 6); value i of a unit is
 *   bits [b*i, b*i+b) of the little-endian integer formed by the unit's bytes.
 * QP_LAYOUT_DEVICE: the canonical packing of reordered codes, with its bytes moved to a
 *   tile order (units stay whole).
 *   1. Inside each packing group of G values, packed position p < G/2 holds value 2p and
 *      position G/2 + p holds value 2p + 1, so the two values of every pair are G/2*b bits
 *      apart.  Groups: 4 consecutive k (6-bit), 8 consecutive k (3-, 4-, 5-bit), the two
 *      8-k blocks at k0 and k0 + 32 with k0 % 64 < 32 (2-bit, 16 values).
 *   2. Canonical unit packing of the reordered codes (as QP_LAYOUT_CANONICAL).
 *   3. 16-row x 256-k tiles (row-block major, then k-tile; 512*b bytes per tile).  In a tile,
 *      lane l = 16*t + r (r = row in the block, t = 0..3) owns a chunk of eight 8-k blocks
 *      of row r -- block j (0..7) starts at k0 = 256*kt + 128*(j/4) + 32*(j%4) + 8*t and is
 *      b bytes -- and chunk byte c is stored at 1024*(c/16) + 16*l + c%16 while
 *      c < F = 16*floor(b/2), else at 64*F + 8*l + (c-F).
 *   Each lane's chunk is what one wave lane feeds to eight 16x16x32 matrix-core steps; one
 *   mask extracts a pair of values as an fp16 pair.  Requires n % 16 == 0, k % 256 == 0. */
enum { QP_LAYOUT_CANONICAL = 0, QP_LAYOUT_DEVICE = 1 };

/* Epilogues of qlinear_grouped_gemm. */
enum {
    QP_EPI_NONE = 0,    /* y[r][n] = fp16(acc)                                        */
    QP_EPI_SWIGLU = 1,  /* rows are gate/up blocks interleaved by 16 (see below);
                           y[r][j] = fp16(silu(gate_j) * up_j), j < n/2                */
    QP_EPI_ROWS_F32 = 2 /* y is float: y[r][n] = acc (fp32), for a later combine      */
};

/* Zero points of the groups.
 *  QP_ZERO_STORED:   affine groups; one u8 zero point per group in qp_weight.zeros
 *                    (inference acceleration guide, s1.1).
 *  QP_ZERO_MIDPOINT: symmetric groups (mixed-bit page, s2.3: the zero point dropped at 2 and
 *                    3 bits, the scale absorbing the offset): the group range is [-m, m] with
 *                    m = max |w|, scale = fp16((m + m) / (2^b - 1)), and the zero point is the
 *                    midpoint 2^(b-1), implied rather than stored (qp_weight.zeros is not read
 *                    and may be NULL).  An all-zero group gets scale 1.0 with every code at
 *                    the midpoint.  Allowed at every bit width.
 *  QP_ZERO_PACKED:   affine groups as QP_ZERO_STORED, with the zero points kept in b bits
 *                    (mixed-bit page, s2.3: a b-bit group's zero point costs b bits): row n of
 *                    qp_weight.zeros is a little-endian bit stream in which group g's zero point
 *                    occupies bits [g*b, g*b + b), padded to whole 32-bit words
 *                    (qp_zero_bytes(desc) bytes in all).  qpack_quantize writes u8 zero points
 *                    in this mode too; qpack_pack_zeros turns them into the packed form.  Read by
 *                    every matmul. */
enum { QP_ZERO_STORED = 0, QP_ZERO_MIDPOINT = 1, QP_ZERO_PACKED = 2 };

/* Storage of the group scales (qp_weight_desc.scale_format).
 *  QP_SCALE_FP16: one fp16 scale per group in qp_weight.scales.
 *  QP_SCALE_FP8:  8-bit float scales with an fp16 fallback (mixed-bit page, s2.3: 2-bit groups
 *                 of 32 at 2.25 bits per weight, the few blocks out of the fp8 range kept in
 *                 fp16).  Group (n, g) has one byte in qp_weight.scales8 [n][k/g]:
 *                  - bit 7 clear: an E4M3 value (OCP 8-bit float: 4-bit exponent, bias 7, 3-bit
 *                    mantissa; 0x7F is NaN); the scale is row_factors[n] times that value;
 *                  - bit 7 set: the scale is the fp16 fb_scales[n * fb_stride + (byte & 0x7F)].
 *                 Written by qpack_quantize_fp8; read by qlinear_gemv, qlinear_gemv_batch (one
 *                 scale format per batch), qlinear_gemm, qlinear_gemm_a8, qlinear_grouped_gemm,
 *                 qmoe_ffn and qlinear_gemv_host (byte or implied zero points; every problem or
 *                 expert brings its own scale bytes, row factors and fallback list).
 *                 qp_blob_write returns QP_ERR_UNSUPPORTED for it (qp_blob_bytes 0). */
enum { QP_SCALE_FP16 = 0, QP_SCALE_FP8 = 1 };

/* Shape and format of one quantized matrix W[n][k]. */
typedef struct {
    int32_t bits;       /* 2, 3, 4, 5 or 6 */
    int32_t group_size; /* 32, 64 or 128 weights of consecutive k inside a row share a scale and
                           zero point (mixed-bit page, s2.3: small groups for the lowest bit
                           widths).  Every call takes all three, except qlinear_gemm_a8 (128)
                           and qlinear_gemv_batch (one group size per batch). */
    int32_t layout;     /* QP_LAYOUT_CANONICAL or QP_LAYOUT_DEVICE */
    int32_t zero_mode;  /* QP_ZERO_STORED, QP_ZERO_MIDPOINT or QP_ZERO_PACKED */
    int64_t n;          /* rows (output features) */
    int64_t k;          /* columns (input features), multiple of 128 */
    int32_t scale_format; /* QP_SCALE_FP16 (0) or QP_SCALE_FP8 */
    int32_t reserved;     /* 0 */
} qp_weight_desc;

/* Device buffers of one quantized matrix. */
typedef struct {
    const void *packed;         /* qp_packed_bytes(desc) bytes, 16-byte aligned */
    const uint16_t *scales;     /* fp16 [n][k/group_size], row-major (planar), 4-byte aligned */
    const uint8_t *zeros;       /* u8   [n][k/group_size], row-major, 2-byte aligned (QP_ZERO_STORED);
                                   b-bit rows of qp_zero_bytes(desc)/n bytes, 4-byte aligned
                                   (QP_ZERO_PACKED); unused (QP_ZERO_MIDPOINT) */
    const int32_t *csr_rowptr;  /* [n+1] outlier CSR over rows of W, or NULL */
    const int32_t *csr_col;     /* [nnz] column k of each outlier, ascending within a row */
    const uint16_t *csr_val;    /* [nnz] fp16 value of each outlier */
    int64_t nnz;                /* number of outliers (0 if csr_rowptr is NULL) */
    /* QP_SCALE_FP8 only (scales unused; no outlier CSR: csr_rowptr NULL, nnz 0):          */
    const uint8_t *scales8;     /* [n][k/group_size] scale bytes, 4-byte aligned */
    const float *row_factors;   /* [n] fp32 factor of each row's E4M3 scales */
    const uint16_t *fb_scales;  /* [n][fb_stride] fp16 fallback scales (NULL if fb_stride is 0) */
    int64_t fb_stride;          /* fallback slots per row, 0..128 */
} qp_weight;

/* ---- host-side accounting (no device work) ------------------------------------------ */

/* n*k*bits/8, or 0 if desc is invalid. */
size_t qp_packed_bytes(const qp_weight_desc *desc);
/* n*k/group_size, or 0 if desc is invalid. */
size_t qp_num_groups(const qp_weight_desc *desc);
/* Bytes of qp_weight.zeros for desc->zero_mode: n*k/g (stored), n*4*ceil((k/g)*bits/32)
 * (packed), 0 (midpoint); 0 if desc is invalid. */
size_t qp_zero_bytes(const qp_weight_desc *desc);
/* Bytes of `numel` weights at `bits` with one scale of `scale_bytes` and a zero point of
 * `zp_bits` per group of `group`: numel*bits/8 + (numel/group)*(scale_bytes + zp_bits/8)
 * (mixed-bit page s2.3; KV page s3.1). */
double qp_quant_bytes(double numel, double bits, double group, double scale_bytes,
                      double zp_bits);
/* Number of held-out outliers for a fraction of an n x k matrix: floor(frac * n * k)
 * computed in double (0 for frac <= 0). */
int64_t qp_outlier_count(int64_t n, int64_t k, double frac);

/* ---- quantize and pack -------------------------------------------------------------- */

/* Scratch bytes qpack_quantize needs for this shape and outlier fraction (0 if none). */
size_t qpack_quantize_workspace_bytes(const qp_weight_desc *desc, double outlier_frac);

/*
 * Group quantizer (inference-acceleration page s1.1; 70B page s2).
 *  w        fp16 [n][ldw] device, ldw >= k, ldw even, 4-byte aligned.
 *  outlier_frac  0 for none; else the floor(frac*n*k) largest |w| (fp16 magnitude, ties to
 *           the lower row-major index) are held out: their dense slot becomes +0 before
 *           the group range is taken, and the original values go to the CSR.
 *  codes    u8 [n][k] device (one code per byte, unpacked).
 *  scales   fp16 [n][k/g], zeros u8 [n][k/g] device (zeros unused, may be NULL, with
 *           QP_ZERO_MIDPOINT); g = desc->group_size.
 *  csr_rowptr [n+1], csr_col [csr_cap], csr_val [csr_cap] device; may be NULL when
 *           outlier_frac == 0 (csr_rowptr, if given, is then filled with zeros).
 *  nnz_out  HOST pointer, receives the outlier count (also when QP_ERR_WORKSPACE is
 *           returned because csr_cap is too small).
 *  workspace/ws_bytes  device scratch of at least qpack_quantize_workspace_bytes().
 * Per group: lo = min(min w, 0), hi = max(max w, 0); all-zero group -> s = 1, zp = 0;
 * s = fp16_rne((hi-lo)/qmax) in IEEE fp32, raised to 2^-14 if it is zero or subnormal;
 * zp = clamp(-rint(lo/s), 0, qmax); q = clamp(rint(w/s) + zp, 0, qmax) (ties to even).
 * Layout of desc is ignored.  Bit-exact with the CPU reference.
 */
qp_status qpack_quantize(const qp_weight_desc *desc, const uint16_t *w, int64_t ldw,
                         double outlier_frac, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, int32_t *csr_rowptr, int32_t *csr_col,
                         uint16_t *csr_val, int64_t csr_cap, int64_t *nnz_out,
                         void *workspace, size_t ws_bytes, void *stream);

/*
 * Group quantizer with fp8 scales (QP_SCALE_FP8; mixed-bit page, s2.3), no outliers.  Per row:
 * every group's fp32 scale s32 as in qpack_quantize (before its fp16 rounding), the row factor
 * F = (largest s32 of the row's non-zero groups) * 2^-8 (exact: that group maps to 256; 1.0 for
 * an all-zero row), then per group t = s32 / F (IEEE fp32) and
 *  - t >= 2^-6: byte = the smallest E4M3 value >= t (so the range still fits), stored scale
 *    F * value (fp32);
 *  - t < 2^-6 (below E4M3's normal range): byte = 0x80 | j for the row's j-th such group, the
 *    stored scale is the fp16 scale qpack_quantize would give it (fb_scales[n][j]);
 *  - an all-zero group: byte 0, codes at the zero point (0, or the midpoint).
 * Zero points and codes then follow qpack_quantize's formulas with the stored scale.
 *  desc     scale_format QP_SCALE_FP8, zero_mode QP_ZERO_STORED or QP_ZERO_MIDPOINT.
 *  w, ldw, codes, zeros  as in qpack_quantize.
 *  scales8  u8 [n][k/g]; row_factors float [n]; fb_scales u16 [n][fb_stride] (may be NULL when
 *           fb_stride is 0); counts int32 [n] receives each row's number of fallback groups.
 *           A row with more than fb_stride (<= 128) fallbacks keeps only the first fb_stride
 *           (check counts; quantize again with a larger stride).  All device pointers.
 * Bit-exact with the CPU reference.
 */
qp_status qpack_quantize_fp8(const qp_weight_desc *desc, const uint16_t *w, int64_t ldw, uint8_t *codes,
                             uint8_t *scales8, uint8_t *zeros, float *row_factors, uint16_t *fb_scales,
                             int64_t fb_stride, int32_t *counts, void *stream);

/* codes u8 [n][k] (values < 2^bits) -> packed bytes in desc->layout
 * (qp_packed_bytes(desc) bytes, 16-byte aligned). */
qp_status qpack_pack(const qp_weight_desc *desc, const uint8_t *codes, void *packed,
                     void *stream);

/* u8 zero points [n][k/g] (as qpack_quantize writes them, 2-byte aligned) -> the b-bit rows
 * of QP_ZERO_PACKED (qp_zero_bytes(desc) bytes, 4-byte aligned).  desc->zero_mode must be
 * QP_ZERO_PACKED; values must be below 2^bits (they are, from qpack_quantize). */
qp_status qpack_pack_zeros(const qp_weight_desc *desc, const uint8_t *zeros, void *packed_zeros,
                           void *stream);

/* Inverse of qpack_pack: packed bytes in desc->layout -> codes u8 [n][k]. */
qp_status qpack_unpack(const qp_weight_desc *desc, const void *packed, uint8_t *codes,
                       void *stream);

/* ---- matmuls ------------------------------------------------------------------------ */

/*
 * Decode GEMV, 1 <= m <= 16 (fused dequant: 70B page s3; fp32 scale: mixed-bit page s4.2).
 *  desc->layout must be QP_LAYOUT_DEVICE.
 *  x  fp16 [m][ldx] device, ldx >= k, ldx % 8 == 0, 16-byte aligned.
 *  y  fp16 [m][ldy] device, ldy >= n, ldy % 4 == 0, 8-byte aligned.
 *  The optional CSR of `w` is added in fp32 before the single fp16 rounding of y.
 *  QP_SCALE_FP8: each group's fp32 sum is multiplied by its E4M3 value (a fallback group: by
 *  its fp16 scale over the row factor) and the row's sum by the row factor, before the CSR.
 *  A fallback byte 0x80 | j with j >= fb_stride is malformed; it reads the row's last slot
 *  (0 when fb_stride is 0), so the call stays inside the buffers.
 * Returns QP_ERR_UNSUPPORTED for m > 16 (use qlinear_gemm).
 */
qp_status qlinear_gemv(const qp_weight_desc *desc, const qp_weight *w, const uint16_t *x,
                       int64_t ldx, int64_t m, uint16_t *y, int64_t ldy, void *stream);

/*
 * Independent decode GEMVs of one layer in a single launch, e.g. the q/k/v or gate/up
 * projections that read the same activations, each at its own bit width (the mixed-bit page
 * assigns bit widths per projection, s2.2).  Each problem has the operands and result of
 * qlinear_gemv and is validated the same way; `problems` is a HOST array of 1..8 entries.
 * All problems share the group size, the zero-point storage (bytes or implied, or b-bit) and
 * the scale format (QP_ERR_UNSUPPORTED otherwise).  Outputs must not overlap (not checked).
 * Returns the first failing problem's status.
 */
typedef struct {
    qp_weight_desc desc;
    qp_weight w;
    const uint16_t *x;
    int64_t ldx;
    int64_t m;
    uint16_t *y;
    int64_t ldy;
} qp_gemv_problem;
qp_status qlinear_gemv_batch(const qp_gemv_problem *problems, int32_t count, void *stream);

/*
 * Prefill dequant-GEMM for any m >= 1 (tuned for m >= 64): same operands and result as
 * qlinear_gemv, for every group size (32, 64, 128), zero mode and scale format.  Tiles of the
 * packed weight are unpacked in registers and fed to fp16 matrix cores with fp32 accumulation;
 * scales are applied per group in fp32 (QP_SCALE_FP8: the row factor times the E4M3 value,
 * rounded once in fp32 as the quantizer stores it, or the fallback's fp16 scale; a fallback
 * index past the list reads its last slot, 0 for an empty list).
 *  workspace/ws_bytes  device scratch, 16-byte aligned; qlinear_gemm_workspace_bytes(desc, m,
 *           w->nnz) bytes (0 for a dense weight whose output fills the GPU: NULL/0 then).
 *           Parts, in order: with outliers, x transposed (k * ldt fp16) and the fp32 outlier
 *           partial (n * ldt floats), ldt = m rounded up to 128, i.e. (2k + 4n) * ldt bytes
 *           (required); then, for shapes whose 256 x 128 output tiles fill at most half of
 *           the GPU's 256 CUs, the fp32 partials of S = 2, 4 or 8 k parts (4 * S * m * n bytes,
 *           at the next multiple of 256): with them the GEMM splits k into S parts and a
 *           second pass sums the parts (in part order) and the outlier partial before the one
 *           fp16 rounding.  A workspace without that part runs the GEMM unsplit.
 *  Limits: x, the packed weight, and each workspace part under 2 GiB.
 */
size_t qlinear_gemm_workspace_bytes(const qp_weight_desc *desc, int64_t m, int64_t nnz);
qp_status qlinear_gemm(const qp_weight_desc *desc, const qp_weight *w, const uint16_t *x,
                       int64_t ldx, int64_t m, uint16_t *y, int64_t ldy, void *workspace,
                       size_t ws_bytes, void *stream);

/*
 * Dynamic per-token int8 activations for the integer-dot path (W8A8 on the integer matrix
 * units with per-token activation quantization: "大模型推理加速实战：量化、投机采样与PD分离的工程
 * 指南", s1.2 and s3.5).  Row m of x: a = max_k |x[m][k]|, s = a / 127, and
 * xq[m][k] = clamp(rint(x[m][k] / s), -127, 127), every step one IEEE fp32 operation (correctly
 * rounded division, round half to even); an all-zero row gets s = 0 and xq = 0.
 *  x        fp16 [m][ldx] device, ldx >= k, ldx % 8 == 0, 16-byte aligned; finite.
 *  k        multiple of 128.
 *  xq       int8 [m][k] device (row stride k), 8-byte aligned, in the int8 storage map: inside
 *           each 128-k group of a row, 16-byte piece 4s + t (s = 0, 1; t = 0..3) holds
 *           k = 64s + 8t .. 64s + 8t + 7 followed by k = 64s + 32 + 8t .. 64s + 32 + 8t + 7
 *           (one piece is the 16 k one lane feeds to one int8 matrix-core step).
 *  x_scales float [m] device: s per row.
 * m >= 1.
 */
qp_status qact_quantize(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int8_t *xq,
                        float *x_scales, void *stream);

/*
 * Integer-dot dequant-GEMM on int8 activations (the W8A8 path above; mixed-bit page s4.2:
 * codes unpacked to 8-bit integers, integer dot products, the scale applied in fp32):
 *     y[m][n] = fp16( x_scales[m] * sum_g s[n][g] * sum_{k in g} xq[m][k] * (q[n][k] - zp[n][g]) )
 * with each group's integer sum exact (int32) and the sum over groups in fp32.
 *  desc     QP_LAYOUT_DEVICE, group_size 128, any zero mode (stored, implied midpoint, b-bit),
 *           fp16 or fp8 scales (fp8: each group's fp32 sum times its E4M3 value, the row
 *           factor once per output, or the fallback's fp16 scale).
 *  w        no outliers (w->nnz must be 0: the held-out weights are defined against the fp16
 *           activations; use qlinear_gemm for them).
 *  xq, x_scales  from qact_quantize (xq 16-byte aligned, m * k < 2^31).
 *  y        fp16 [m][ldy] device, ldy >= n, ldy % 4 == 0, 8-byte aligned.
 * m >= 1 (as every matmul here).  Returns QP_ERR_UNSUPPORTED for groups of 32 or 64 and for
 * outliers.
 */
qp_status qlinear_gemm_a8(const qp_weight_desc *desc, const qp_weight *w, const int8_t *xq,
                          const float *x_scales, int64_t m, uint16_t *y, int64_t ldy,
                          void *stream);

/*
 * Grouped dequant-GEMM over routed experts (MoE page s4.2).  All experts share `desc`
 * (layout QP_LAYOUT_DEVICE; any group size and zero mode).  `experts` is a HOST array of
 * n_experts (<= 64) weights.
 *  row_src         int32 [rows] device: token (row of x) feeding sorted row r.
 *  expert_offsets  int32 [n_experts+1] device, non-decreasing, from >= 0 to <= rows: rows
 *                  of expert e are [expert_offsets[e], expert_offsets[e+1]).
 *  rows            host upper bound on expert_offsets[n_experts].  It sizes the launch:
 *                  one workgroup per weight tile and per row tile that some routing of
 *                  `rows` rows could occupy; the tiles the routing leaves empty return
 *                  at once.
 *  epilogue        QP_EPI_NONE: y fp16 [rows][ldy];
 *                  QP_EPI_SWIGLU: row blocks 2i and 2i+1 of each expert matrix hold gate
 *                  rows 16i..16i+15 and up rows 16i..16i+15; y fp16 [rows][ldy] gets
 *                  silu(gate)*up for n/2 columns (n % 32 == 0);
 *                  QP_EPI_ROWS_F32: y is float [rows][ldy].
 * Experts with no rows cost no weight traffic.
 */
qp_status qlinear_grouped_gemm(const qp_weight_desc *desc, const qp_weight *experts,
                               int32_t n_experts, const uint16_t *x, int64_t ldx,
                               const int32_t *row_src, const int32_t *expert_offsets,
                               int64_t rows, int32_t epilogue, void *y, int64_t ldy,
                               void *stream);

/* ---- routed-expert plumbing (MoE page s4.2) ----------------------------------------- */

/*
 * Sort the tokens' top-k choices by expert (stable in token, then choice order).
 *  topk_ids   int32 [tokens][topk] device, values in [0, n_experts).
 *  topk_w     float [tokens][topk] device, combine weights.
 *  expert_offsets int32 [n_experts+1], row_src int32 [tokens*topk],
 *  row_weight float [tokens*topk], token_rows int32 [tokens][topk] (sorted row of each
 *  choice) -- all device outputs.  tokens*topk <= 65536, n_experts <= 64.
 */
qp_status qmoe_dispatch(const int32_t *topk_ids, const float *topk_w, int64_t tokens,
                        int32_t topk, int32_t n_experts, int32_t *expert_offsets,
                        int32_t *row_src, float *row_weight, int32_t *token_rows,
                        void *stream);

/*
 * out[t][j] = fp16( sum_{c < topk} row_weight[r_c] * rows_f32[r_c][j] ), r_c =
 * token_rows[t][c], summed in fp32 in choice order (deterministic, no atomics).
 *  rows_f32 float [*][ld_rows], out fp16 [tokens][ldo], n columns.
 */
qp_status qmoe_combine(const float *rows_f32, int64_t ld_rows, const int32_t *token_rows,
                       const float *row_weight, int64_t tokens, int32_t topk, int64_t n,
                       uint16_t *out, int64_t ldo, void *stream);

/* Scratch bytes of qmoe_ffn. */
size_t qmoe_ffn_workspace_bytes(int64_t tokens, int32_t topk, int32_t n_experts,
                                int64_t d_model, int64_t d_ff);

/*
 * Whole routed-expert FFN on one stream: dispatch, grouped gate/up GEMM with SwiGLU
 * (intermediate stored in fp16), grouped down GEMM (fp32 rows), weighted combine.
 *  gate_up[e]: desc_gu = {bits, g, DEVICE, zero mode, 2*d_ff, d_model}, gate/up rows
 *              interleaved in blocks of 16 (see QP_EPI_SWIGLU);  down[e]: desc_d = {.., d_model,
 *              d_ff}, with the same bit width (group size and zero mode may differ).
 *  x fp16 [tokens][ldx]; out fp16 [tokens][ldo]; HOST arrays gate_up/down.
 */
qp_status qmoe_ffn(const qp_weight_desc *desc_gu, const qp_weight *gate_up,
                   const qp_weight_desc *desc_d, const qp_weight *down, int32_t n_experts,
                   const uint16_t *x, int64_t ldx, int64_t tokens, const int32_t *topk_ids,
                   const float *topk_w, int32_t topk, uint16_t *out, int64_t ldo,
                   void *workspace, size_t ws_bytes, void *stream);

/* ---- quantized KV cache and decode attention (KV-cache quantization page, kwkr.cn) ---- */

/*
 * Geometry and format of a quantized KV cache.  Each (sequence b, kv head h) owns
 * `capacity` token slots; cache row R = (b*kv_heads + h)*capacity + token.  K and V are
 * quantized per row in symmetric groups of adjacent head-dimension values (s2.1, s2.2) at
 * their own bit widths (s2.3: INT4 K with INT8 V is the page's middle ground) with one fp32
 * scale per group (s3.1):
 *     m = max |x| over the group, qmax = 2^(bits-1) - 1, s = m / qmax (IEEE fp32),
 *     q = clamp(rint(x / s), -qmax, qmax) (ties to even), stored as q + 2^(bits-1);
 *     an all-zero group stores s = 0 and q = 0.
 * Code bytes (4-bit values two per byte, s5.1; value p is the low nibble of byte p/2 when p
 * is even; sigma(s) = s at 8 bits, s/2 + 4*(s%2) at 4 bits):
 *   K  row R holds 128*k_bits/8 bytes; value d = 32j + 8t + s sits at 32t + 8j + sigma(s).
 *   V  each (b, h) holds capacity/32 tiles of 32 tokens (32*128*v_bits/8 bytes each); token
 *      w of a tile, w = 4t + s (s < 4) or 16 + 4t + s - 4 (s >= 4), value d = 16c + r, sits
 *      at 64*P*(c/(P/8)) + P*(16t + r) + 8*(c%(P/8)) + sigma(s), P = 128/v_bits.
 *   Scales: fp32 [rows][128/group].
 * These orders put every operand of the attention's 16x16x32 matrix-core steps in one
 * contiguous 16-64 byte piece per lane.
 */
typedef struct {
    int32_t batch;      /* sequences */
    int32_t q_heads;    /* query heads, a multiple of kv_heads with q_heads/kv_heads <= 16 */
    int32_t kv_heads;
    int32_t head_dim;   /* 128 */
    int32_t k_bits;     /* 4 or 8 */
    int32_t v_bits;     /* 4 or 8 */
    int32_t k_group;    /* 32, 64 or 128 */
    int32_t v_group;    /* 32, 64 or 128 */
    int64_t capacity;   /* token slots per (sequence, kv head): a multiple of 32, < 2^24 */
} qkv_desc;
enum { QKV_K = 0, QKV_V = 1 };

/* Code bytes of the whole K (which = QKV_K) or V cache: batch*kv_heads*capacity*128*bits/8,
 * or 0 if desc is invalid. */
size_t qkv_cache_bytes(const qkv_desc *desc, int32_t which);
/* fp32 scales of the whole K or V cache: batch*kv_heads*capacity*128/group (0 if invalid). */
size_t qkv_scale_count(const qkv_desc *desc, int32_t which);

/*
 * Quantize `rows` new K (or V) head vectors into the cache (the write path of a decode or
 * prefill step).
 *  x       fp16 [rows][ldx] device, ldx >= 128, ldx % 8 == 0, 16-byte aligned.
 *  slots   int64 [rows] device: cache row R of each input row.  Rows whose slot is outside
 *          [0, batch*kv_heads*capacity) are skipped (the device cannot report them).
 *          Slots must be distinct within one call.
 *  codes   the cache's code bytes (qkv_cache_bytes), 16-byte aligned; scales fp32
 *          (qkv_scale_count), 16-byte aligned.  Only the addressed rows change.
 * Bit-exact with the CPU reference.
 */
qp_status qkv_quantize(const qkv_desc *desc, int32_t which, const uint16_t *x, int64_t ldx,
                       const int64_t *slots, int64_t rows, void *codes, float *scales,
                       void *stream);

/* Scratch bytes of qattn_decode (0 when one chunk per (sequence, kv head) suffices). */
size_t qattn_decode_workspace_bytes(const qkv_desc *desc);

/*
 * Decode attention over the quantized cache, one query token per sequence (s5.1: the
 * operator reads the packed codes and scales and dequantizes in registers).  For sequence
 * b and query head h (kv head h / (q_heads/kv_heads)), over its first seq_lens[b] tokens:
 *     z_t = sm_scale * q[b][h] . K_t,   p = softmax(z),   o[b][h] = sum_t p_t V_t
 * with K_t, V_t the dequantized rows (code - 2^(bits-1)) * scale.  Scores accumulate in
 * fp32 (each K group scaled in fp32); V values are dequantized to fp16 and the softmax
 * weights (at most 2^14 times their share) are rounded to fp16 for the matrix cores; o is
 * rounded once to fp16.  seq_lens[b] <= 0 gives o = 0; lengths above capacity are clamped.
 *  q        fp16 [batch][q_heads][128] device, 16-byte aligned.
 *  seq_lens int32 [batch] device.
 *  o        fp16 [batch][q_heads][128] device.
 *  workspace/ws_bytes  at least qattn_decode_workspace_bytes(desc) bytes, 16-byte aligned.
 */
qp_status qattn_decode(const qkv_desc *desc, const uint16_t *q, const void *k_codes,
                       const float *k_scales, const void *v_codes, const float *v_scales,
                       const int32_t *seq_lens, float sm_scale, uint16_t *o, void *workspace,
                       size_t ws_bytes, void *stream);

/*
 * qattn_decode for callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results as qattn_decode, without the workspace: the chunk partials live in a fixed array
 * inside the library, QATTN_NOALLOC_SCRATCH_BYTES bytes per GPU, created with the library and
 * held by each GPU it runs on until the process ends.  Its address on a GPU is looked up once,
 * on the first call with that GPU current.  No call allocates anything.
 *  Limit: qattn_decode_workspace_bytes(desc) must not exceed QATTN_NOALLOC_SCRATCH_BYTES
 *  (2 MiB covers every shape with up to 8 query heads per kv head, and more whenever the
 *  cache is split into fewer chunks); otherwise QP_ERR_WORKSPACE and nothing is launched.
 *  All calls on one GPU share the array: calls that overlap on one GPU (different streams,
 *  or host threads without ordering) race and give wrong results.  The array is written
 *  before it is read within a call, so nothing needs clearing between calls.
 */
#define QATTN_NOALLOC_SCRATCH_BYTES (2u * 1024u * 1024u)
qp_status qattn_decode_noalloc(const qkv_desc *desc, const uint16_t *q, const void *k_codes,
                               const float *k_scales, const void *v_codes, const float *v_scales,
                               const int32_t *seq_lens, float sm_scale, uint16_t *o, void *stream);

/*
 * Decode GEMV on the HOST CPU for a CPU/GPU layer split (the CPU half of the 2/3/5/6-bit mixed
 * quantization page: s4.1 fused unpack and multiply-accumulate ordered by output, no buffer of
 * unpacked weights, byte-permute unpacking on 256-bit vectors; s4.3 prefetch distance 4; s5.2
 * one core left to the scheduling side).  Same result definition as qlinear_gemv:
 *     y[m][n] = fp16( sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - zp[n][g])
 *                     + sum_{CSR row n} x[m][k] * val )
 * accumulated in fp32 (each group's partial, then its scale, then the outliers, in fp32).
 *  desc     canonical layout (QP_LAYOUT_CANONICAL), groups of 32/64/128, byte or implied zero
 *           points (QP_ZERO_STORED / QP_ZERO_MIDPOINT), fp16 or fp8 scales (a group's fp8
 *           scale is the row factor times its E4M3 value in fp32, or its fp16 fallback).
 *  w        HOST pointers: packed canonical rows, scales (or scales8, row_factors and the
 *           fallback list), zeros, optional CSR (fp16 scales only).
 *  x, y     HOST fp16 [m][ldx] and [m][ldy]; 1 <= m <= 8.
 *  threads  worker threads (OpenMP); 0 = the machine's processors minus one.
 * Three code paths, chosen at run time from the CPU's features: AVX-512 with byte permutes
 * (F, BW, VL, VBMI: 16 codes per 512-bit vector, each decoded straight to the fp32 value
 * 1 + q/2^b), else AVX2/FMA/F16C (8 codes per 256-bit vector), else a portable loop.  They
 * sum in different orders (fp32 results agree to rounding, not bit for bit).  The environment
 * variables QPACK_HOST_AVX2 and QPACK_HOST_PORTABLE force the lesser paths.
 * Synchronous; allocates nothing.
 */
qp_status qlinear_gemv_host(const qp_weight_desc *desc, const qp_weight *w, const uint16_t *x, int64_t ldx,
                            int64_t m, uint16_t *y, int64_t ldy, int32_t threads);
/* The path qlinear_gemv_host takes on this host now: "avx512vbmi", "avx2" or "portable"
 * (a static string). */
const char *qlinear_gemv_host_isa(void);

/*
 * Serialized packed weight (HOST memory): a self-describing little-endian byte string holding
 * one quantized, packed weight -- codes (either layout), scales, zero points and the outlier
 * CSR -- so a repacked model can be stored and reloaded without repacking (the one-time repack
 * of the single-GPU 70B page, s3; every field little-endian as the mixed-bit page, s3.2, reads
 * its units).  Layout: a 64-byte header -- "QPKW", u32 version 1, u32 header size 64, i32 bits,
 * i32 group size, i32 layout, i32 zero mode, u32 flags 0, i64 n, i64 k, i64 nnz, u32 CRC-32
 * (IEEE) of the whole blob with this field counted as zeros, u32 0 -- then sections at
 * multiples of 64 bytes:
 * packed codes, scales (u16 each), zero points (absent for implied ones), and with nnz > 0 the
 * CSR row pointers (i32, n+1), columns (i32) and values (u16).
 */
/* Bytes of the blob of a weight with `nnz` outliers (0 if desc is invalid). */
size_t qp_blob_bytes(const qp_weight_desc *desc, int64_t nnz);
/* Serialize.  w holds HOST pointers (sizes as for the device arrays; CSR arrays only when
 * w->nnz > 0).  blob: host, at least qp_blob_bytes(desc, w->nnz) bytes (else QP_ERR_WORKSPACE). */
qp_status qp_blob_write(const qp_weight_desc *desc, const qp_weight *w, void *blob, size_t blob_bytes);
/* Check a blob (magic, version, sizes, checksum, CSR row pointers and columns) and return its
 * descriptor, its nnz and, if offsets is not NULL, the byte offsets of its six sections
 * (packed, scales, zeros, rowptr, col, val; 0 for an absent section).  The sections hold
 * little-endian integers and can be used in place on a little-endian host.  A blob that
 * fails any check returns QP_ERR_INVALID_ARG (QP_ERR_UNSUPPORTED for an unknown version). */
qp_status qp_blob_parse(const void *blob, size_t blob_bytes, qp_weight_desc *desc_out, int64_t *nnz_out,
                        size_t *offsets);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *qp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QPACK_H */
