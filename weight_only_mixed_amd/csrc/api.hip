// C-ABI entry points of libqpack: argument validation on the host, then kernel launches.
// Nothing is launched or written unless every argument passes validation.  See qpack.h for
// the contract of each call and the passages of the pages it follows.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kv_internal.h"
#include "qp_internal.h"

namespace qp {

static thread_local char g_err[512];

qp_status fail(qp_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

static qp_status ok()
{
    g_err[0] = 0;
    return QP_OK;
}

static qp_status device(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(QP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// a * b * c > lim, for non-negative factors, without overflowing.
static bool prod_over(int64_t a, int64_t b, int64_t c, int64_t lim)
{
    int64_t ab, abc;
    if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc)) return true;
    return abc > lim;
}

// Shape/format checks shared by every call.  need_device: layout must be DEVICE.
static qp_status check_desc(const qp_weight_desc *d, bool need_device)
{
    if (!d) return fail(QP_ERR_INVALID_ARG, "desc is NULL");
    if (d->bits < 2 || d->bits > 6) return fail(QP_ERR_INVALID_ARG, "bits=%d not in 2..6", d->bits);
    if (d->zero_mode != QP_ZERO_STORED && d->zero_mode != QP_ZERO_MIDPOINT && d->zero_mode != QP_ZERO_PACKED)
        return fail(QP_ERR_INVALID_ARG, "zero_mode=%d unknown", d->zero_mode);
    if (d->layout != QP_LAYOUT_CANONICAL && d->layout != QP_LAYOUT_DEVICE)
        return fail(QP_ERR_INVALID_ARG, "layout=%d unknown", d->layout);
    if (d->n <= 0 || d->k <= 0) return fail(QP_ERR_INVALID_ARG, "n=%lld k=%lld must be > 0", (long long)d->n, (long long)d->k);
    if (d->group_size <= 0 || d->k % d->group_size != 0)
        return fail(QP_ERR_INVALID_ARG, "k=%lld not a multiple of group_size=%d", (long long)d->k, d->group_size);
    if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128)
        return fail(QP_ERR_UNSUPPORTED, "group_size=%d (32, 64 and 128 are built)", d->group_size);
    if (d->k % 128 != 0) return fail(QP_ERR_UNSUPPORTED, "k=%lld must be a multiple of 128", (long long)d->k);
    if (d->n > (1LL << 31) - 1 || prod_over(d->n, d->k, 1, 1LL << 40))
        return fail(QP_ERR_INVALID_ARG, "matrix too large");
    if (d->layout == QP_LAYOUT_DEVICE && (d->n % kTileN != 0 || d->k % kTileK != 0))
        return fail(QP_ERR_INVALID_ARG, "device layout needs n %% 16 == 0 and k %% 256 == 0 (n=%lld k=%lld)",
                    (long long)d->n, (long long)d->k);
    if (need_device && d->layout != QP_LAYOUT_DEVICE)
        return fail(QP_ERR_UNSUPPORTED, "matmuls read the device layout (pack with QP_LAYOUT_DEVICE)");
    if (d->scale_format != QP_SCALE_FP16 && d->scale_format != QP_SCALE_FP8)
        return fail(QP_ERR_INVALID_ARG, "scale_format=%d unknown", d->scale_format);
    if (d->scale_format == QP_SCALE_FP8 && d->zero_mode == QP_ZERO_PACKED)
        return fail(QP_ERR_UNSUPPORTED, "fp8 scales take byte or implied zero points");
    return QP_OK;
}

// Calls that read only fp16 scales.
static qp_status need_fp16_scales(const qp_weight_desc *d, const char *who)
{
    if (d->scale_format != QP_SCALE_FP16)
        return fail(QP_ERR_UNSUPPORTED,
                    "%s reads fp16 scales (fp8 scales: qpack_quantize_fp8 writes them, every matmul reads them)",
                    who);
    return QP_OK;
}

// The kernels' view of a validated weight: with fp8 scales, `scales` carries the scale bytes
// and the row factors and fallback list ride along.
static ExpertPtrs weight_ptrs(const qp_weight_desc *d, const qp_weight *w)
{
    if (d->scale_format == QP_SCALE_FP8)
        return {(const uint8_t *)w->packed, (const uint16_t *)w->scales8, w->zeros, w->row_factors,
                w->fb_stride > 0 ? w->fb_scales : nullptr, (int32_t)w->fb_stride};
    return {(const uint8_t *)w->packed, w->scales, w->zeros, nullptr, nullptr, 0};
}

static qp_status check_weight(const qp_weight_desc *d, const qp_weight *w, bool allow_csr)
{
    if (!w) return fail(QP_ERR_INVALID_ARG, "weight is NULL");
    if (!w->packed || !aligned(w->packed, 16)) return fail(QP_ERR_INVALID_ARG, "packed NULL or not 16-byte aligned");
    if (d->scale_format == QP_SCALE_FP8) {
        if (!w->scales8 || !aligned(w->scales8, 4)) return fail(QP_ERR_INVALID_ARG, "scales8 NULL or not 4-byte aligned");
        if (!w->row_factors || !aligned(w->row_factors, 4))
            return fail(QP_ERR_INVALID_ARG, "row_factors NULL or not 4-byte aligned");
        if (w->fb_stride < 0 || w->fb_stride > 128)
            return fail(QP_ERR_INVALID_ARG, "fb_stride=%lld not in 0..128", (long long)w->fb_stride);
        if (w->fb_stride > 0 && (!w->fb_scales || !aligned(w->fb_scales, 2)))
            return fail(QP_ERR_INVALID_ARG, "fb_scales NULL or not 2-byte aligned");
        if (w->nnz != 0 || w->csr_rowptr)
            return fail(QP_ERR_UNSUPPORTED, "fp8-scale weights carry no outlier CSR (qpack_quantize_fp8 holds none out)");
    } else if (!w->scales || !aligned(w->scales, 4)) {
        return fail(QP_ERR_INVALID_ARG, "scales NULL or not 4-byte aligned");
    }
    if (d->zero_mode == QP_ZERO_STORED && (!w->zeros || !aligned(w->zeros, 2)))
        return fail(QP_ERR_INVALID_ARG, "zeros NULL or not 2-byte aligned");
    if (d->zero_mode == QP_ZERO_PACKED && (!w->zeros || !aligned(w->zeros, 4)))
        return fail(QP_ERR_INVALID_ARG, "packed zeros NULL or not 4-byte aligned");
    if (w->nnz < 0) return fail(QP_ERR_INVALID_ARG, "nnz < 0");
    if (w->csr_rowptr) {
        if (!allow_csr && w->nnz > 0) return fail(QP_ERR_UNSUPPORTED, "outlier CSR not supported here");
        if (w->nnz > 0 && (!w->csr_col || !w->csr_val)) return fail(QP_ERR_INVALID_ARG, "CSR col/val NULL with nnz > 0");
    } else if (w->nnz > 0) {
        return fail(QP_ERR_INVALID_ARG, "nnz > 0 but csr_rowptr is NULL");
    }
    return QP_OK;
}

// Zero-point pair the kernels use in place of the stored ones: 0 = read them; for implied
// midpoints, 2^(b-1) in both bytes (a row's two groups of one k-tile).
static uint32_t zero_pair(const qp_weight_desc *d)
{
    return d->zero_mode == QP_ZERO_MIDPOINT ? 0x101u << (d->bits - 1) : 0u;
}

static hipStream_t S(void *s) { return (hipStream_t)s; }

// Bytes of one row of b-bit zero points (QP_ZERO_PACKED): whole 32-bit words.
static int64_t zero_row_bytes(const qp_weight_desc *d)
{
    return 4 * ((d->k / d->group_size * d->bits + 31) / 32);
}

// Geometry of a quantized KV cache (qkv_desc).
static qp_status check_kv(const qkv_desc *d)
{
    if (!d) return fail(QP_ERR_INVALID_ARG, "desc is NULL");
    if (d->head_dim != 128) return fail(QP_ERR_UNSUPPORTED, "head_dim=%d (128 is built)", d->head_dim);
    if ((d->k_bits != 4 && d->k_bits != 8) || (d->v_bits != 4 && d->v_bits != 8))
        return fail(QP_ERR_UNSUPPORTED, "k_bits=%d v_bits=%d (4 and 8 are built)", d->k_bits, d->v_bits);
    for (int g : {d->k_group, d->v_group})
        if (g != 32 && g != 64 && g != 128) return fail(QP_ERR_UNSUPPORTED, "group %d (32, 64, 128 are built)", g);
    if (d->batch < 1 || d->kv_heads < 1 || d->q_heads < 1)
        return fail(QP_ERR_INVALID_ARG, "batch, q_heads and kv_heads must be >= 1");
    if (d->q_heads % d->kv_heads != 0) return fail(QP_ERR_INVALID_ARG, "q_heads must be a multiple of kv_heads");
    if (d->q_heads / d->kv_heads > 16) return fail(QP_ERR_UNSUPPORTED, "more than 16 query heads per kv head");
    if (d->capacity < 32 || d->capacity % 32 != 0 || d->capacity >= (1LL << 24))
        return fail(QP_ERR_INVALID_ARG, "capacity=%lld must be a multiple of 32 below 2^24", (long long)d->capacity);
    if ((int64_t)d->batch * d->kv_heads > (1LL << 16) || d->batch > 65535 || d->kv_heads > 65535)
        return fail(QP_ERR_INVALID_ARG, "batch*kv_heads above 65536 (or batch or kv_heads above 65535)");
    return QP_OK;
}

static int64_t kv_rows(const qkv_desc *d) { return (int64_t)d->batch * d->kv_heads * d->capacity; }

// Scratch of qattn_decode_noalloc: one copy per GPU.  In host code `scratch` names a host-side
// stand-in, not device memory, so its device address is looked up per device (with that device
// current) and only that address is ever passed to kernels.
__device__ __align__(256) uint8_t scratch[QATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];

static qp_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QP_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(QP_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QP_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return QP_OK;
}

}  // namespace qp

using namespace qp;

extern "C" {

const char *qp_last_error(void) { return g_err; }

size_t qp_packed_bytes(const qp_weight_desc *d)
{
    if (check_desc(d, false) != QP_OK) return 0;
    return (size_t)(d->n * d->k * d->bits / 8);
}

size_t qp_num_groups(const qp_weight_desc *d)
{
    if (check_desc(d, false) != QP_OK) return 0;
    return (size_t)(d->n * (d->k / d->group_size));
}

size_t qp_zero_bytes(const qp_weight_desc *d)
{
    if (check_desc(d, false) != QP_OK) return 0;
    if (d->zero_mode == QP_ZERO_MIDPOINT) return 0;
    if (d->zero_mode == QP_ZERO_PACKED) return (size_t)(d->n * zero_row_bytes(d));
    return (size_t)(d->n * (d->k / d->group_size));
}

double qp_quant_bytes(double numel, double bits, double group, double scale_bytes, double zp_bits)
{
    return numel * bits / 8.0 + (numel / group) * (scale_bytes + zp_bits / 8.0);
}

int64_t qp_outlier_count(int64_t n, int64_t k, double frac)
{
    if (!(frac > 0.0) || n <= 0 || k <= 0) return 0;
    return (int64_t)floor(frac * (double)(n * k));
}

size_t qpack_quantize_workspace_bytes(const qp_weight_desc *d, double outlier_frac)
{
    if (check_desc(d, false) != QP_OK) return 0;
    return qp_outlier_count(d->n, d->k, outlier_frac) > 0 ? quant_ws_bytes(d->n) : 0;
}

qp_status qpack_quantize(const qp_weight_desc *d, const uint16_t *w, int64_t ldw, double outlier_frac,
                         uint8_t *codes, uint16_t *scales, uint8_t *zeros, int32_t *csr_rowptr,
                         int32_t *csr_col, uint16_t *csr_val, int64_t csr_cap, int64_t *nnz_out,
                         void *workspace, size_t ws_bytes, void *stream)
{
    qp_status st = check_desc(d, false);
    if (st != QP_OK) return st;
    if ((st = need_fp16_scales(d, "qpack_quantize")) != QP_OK) return st;
    if (!w || !aligned(w, 4)) return fail(QP_ERR_INVALID_ARG, "w NULL or not 4-byte aligned");
    if (ldw < d->k || ldw % 2 != 0) return fail(QP_ERR_INVALID_ARG, "ldw=%lld must be >= k and even", (long long)ldw);
    if (!codes || !aligned(codes, 2)) return fail(QP_ERR_INVALID_ARG, "codes NULL or not 2-byte aligned");
    if (!scales || (!zeros && d->zero_mode != QP_ZERO_MIDPOINT)) return fail(QP_ERR_INVALID_ARG, "scales/zeros NULL");
    if (!nnz_out) return fail(QP_ERR_INVALID_ARG, "nnz_out NULL");
    if (outlier_frac < 0.0 || outlier_frac > 1.0 || outlier_frac != outlier_frac)
        return fail(QP_ERR_INVALID_ARG, "outlier_frac must be in [0, 1]");
    const int64_t kout = qp_outlier_count(d->n, d->k, outlier_frac);
    if (kout > 0) {
        if (!csr_rowptr || !csr_col || !csr_val) return fail(QP_ERR_INVALID_ARG, "CSR outputs NULL with outliers requested");
        if (d->n * d->k > 0x7FFFFFFFLL) return fail(QP_ERR_UNSUPPORTED, "outliers need n*k < 2^31");
        if (csr_cap < kout) {
            *nnz_out = kout;
            return fail(QP_ERR_WORKSPACE, "csr_cap=%lld < %lld outliers", (long long)csr_cap, (long long)kout);
        }
        const size_t need = quant_ws_bytes(d->n);
        if (!workspace || ws_bytes < need || !aligned(workspace, 16))
            return fail(QP_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
    }
    *nnz_out = kout;
    QuantWs ws{};
    if (kout > 0) ws = quant_ws_carve(workspace, d->n);
    return device(launch_quantize(d->bits, d->zero_mode == QP_ZERO_MIDPOINT, w, ldw, d->n, d->k, d->group_size, kout, codes, scales,
                                  zeros, csr_rowptr, csr_col, csr_val, ws, S(stream)),
                  "qpack_quantize");
}

qp_status qpack_quantize_fp8(const qp_weight_desc *d, const uint16_t *w, int64_t ldw, uint8_t *codes,
                             uint8_t *scales8, uint8_t *zeros, float *row_factors, uint16_t *fb_scales,
                             int64_t fb_stride, int32_t *counts, void *stream)
{
    qp_status st = check_desc(d, false);
    if (st != QP_OK) return st;
    if (d->scale_format != QP_SCALE_FP8) return fail(QP_ERR_INVALID_ARG, "scale_format must be QP_SCALE_FP8");
    if (!w || !aligned(w, 4)) return fail(QP_ERR_INVALID_ARG, "w NULL or not 4-byte aligned");
    if (ldw < d->k || ldw % 2 != 0) return fail(QP_ERR_INVALID_ARG, "ldw=%lld must be >= k and even", (long long)ldw);
    if (!codes || !aligned(codes, 2)) return fail(QP_ERR_INVALID_ARG, "codes NULL or not 2-byte aligned");
    if (!scales8 || !row_factors || !counts) return fail(QP_ERR_INVALID_ARG, "scales8/row_factors/counts NULL");
    if (!aligned(row_factors, 4) || !aligned(counts, 4))
        return fail(QP_ERR_INVALID_ARG, "row_factors/counts not 4-byte aligned");
    if (!zeros && d->zero_mode == QP_ZERO_STORED) return fail(QP_ERR_INVALID_ARG, "zeros NULL");
    if (fb_stride < 0 || fb_stride > 128) return fail(QP_ERR_INVALID_ARG, "fb_stride=%lld not in 0..128", (long long)fb_stride);
    if (fb_stride > 0 && (!fb_scales || !aligned(fb_scales, 2)))
        return fail(QP_ERR_INVALID_ARG, "fb_scales NULL or not 2-byte aligned");
    if (d->k / d->group_size > quantize_fp8_max_groups())
        return fail(QP_ERR_UNSUPPORTED, "k/group_size=%lld above %lld groups per row", (long long)(d->k / d->group_size),
                    (long long)quantize_fp8_max_groups());
    if (d->n > 0x7FFFFFFFLL) return fail(QP_ERR_UNSUPPORTED, "n above 2^31 - 1 rows");
    return device(launch_quantize_fp8(d->bits, d->zero_mode == QP_ZERO_MIDPOINT, w, ldw, d->n, d->k, d->group_size, codes,
                                      scales8, d->zero_mode == QP_ZERO_MIDPOINT ? nullptr : zeros, row_factors,
                                      fb_scales, fb_stride, counts, S(stream)),
                  "qpack_quantize_fp8");
}

qp_status qpack_pack(const qp_weight_desc *d, const uint8_t *codes, void *packed, void *stream)
{
    qp_status st = check_desc(d, false);
    if (st != QP_OK) return st;
    if (!codes || !aligned(codes, 8)) return fail(QP_ERR_INVALID_ARG, "codes NULL or not 8-byte aligned");
    if (!packed || !aligned(packed, 16)) return fail(QP_ERR_INVALID_ARG, "packed NULL or not 16-byte aligned");
    return device(launch_pack(d->bits, d->layout, codes, d->n, d->k, (uint8_t *)packed, S(stream)), "qpack_pack");
}

qp_status qpack_pack_zeros(const qp_weight_desc *d, const uint8_t *zeros, void *packed_zeros, void *stream)
{
    qp_status st = check_desc(d, false);
    if (st != QP_OK) return st;
    if (d->zero_mode != QP_ZERO_PACKED) return fail(QP_ERR_INVALID_ARG, "zero_mode must be QP_ZERO_PACKED");
    if (!zeros || !aligned(zeros, 2)) return fail(QP_ERR_INVALID_ARG, "zeros NULL or not 2-byte aligned");
    if (!packed_zeros || !aligned(packed_zeros, 4)) return fail(QP_ERR_INVALID_ARG, "packed_zeros NULL or not 4-byte aligned");
    return device(launch_pack_zeros(d->bits, zeros, d->n, d->k / d->group_size, zero_row_bytes(d),
                                    (uint8_t *)packed_zeros, S(stream)),
                  "qpack_pack_zeros");
}

qp_status qpack_unpack(const qp_weight_desc *d, const void *packed, uint8_t *codes, void *stream)
{
    qp_status st = check_desc(d, false);
    if (st != QP_OK) return st;
    if (!codes || !aligned(codes, 8)) return fail(QP_ERR_INVALID_ARG, "codes NULL or not 8-byte aligned");
    if (!packed || !aligned(packed, 16)) return fail(QP_ERR_INVALID_ARG, "packed NULL or not 16-byte aligned");
    return device(launch_unpack(d->bits, d->layout, (const uint8_t *)packed, d->n, d->k, codes, S(stream)),
                  "qpack_unpack");
}

static qp_status check_xy(const qp_weight_desc *d, const uint16_t *x, int64_t ldx, int64_t m, const void *y,
                          int64_t ldy, int64_t ncols, size_t ysize)
{
    if (!x || !aligned(x, 16)) return fail(QP_ERR_INVALID_ARG, "x NULL or not 16-byte aligned");
    if (ldx < d->k || ldx % 8 != 0) return fail(QP_ERR_INVALID_ARG, "ldx=%lld must be >= k and a multiple of 8", (long long)ldx);
    if (!y || !aligned(y, 2 * ysize)) return fail(QP_ERR_INVALID_ARG, "y NULL or misaligned");
    if (ldy < ncols || ldy % 4 != 0) return fail(QP_ERR_INVALID_ARG, "ldy=%lld must be >= %lld and a multiple of 4", (long long)ldy, (long long)ncols);
    if (m < 1) return fail(QP_ERR_INVALID_ARG, "m=%lld must be >= 1", (long long)m);
    return QP_OK;
}

// Validated GEMV problem (shared by qlinear_gemv and qlinear_gemv_batch).
static qp_status gemv_problem(const qp_weight_desc *d, const qp_weight *w, const uint16_t *x, int64_t ldx, int64_t m,
                              uint16_t *y, int64_t ldy, GemvProblem *p)
{
    qp_status st = check_desc(d, true);
    if (st != QP_OK) return st;
    if ((st = check_weight(d, w, true)) != QP_OK) return st;
    if ((st = check_xy(d, x, ldx, m, y, ldy, d->n, 4)) != QP_OK) return st;
    if (m > 16) return fail(QP_ERR_UNSUPPORTED, "gemv handles m <= 16 (m=%lld); use qlinear_gemm", (long long)m);
    if (prod_over(m, ldx, 2, 0x7FFFFFFFLL)) return fail(QP_ERR_UNSUPPORTED, "x larger than 2 GiB");
    *p = GemvProblem{};
    p->w = weight_ptrs(d, w);
    p->fp8 = d->scale_format == QP_SCALE_FP8;
    p->zmid = zero_pair(d);
    p->gs = d->group_size;
    p->zrow = d->zero_mode == QP_ZERO_PACKED ? (int32_t)zero_row_bytes(d) : 0;
    if (w->nnz > 0) {
        p->rowptr = w->csr_rowptr;
        p->col = w->csr_col;
        p->val = w->csr_val;
    }
    p->x = x;
    p->ldx = ldx;
    p->m = m;
    p->n = d->n;
    p->k = d->k;
    p->y = y;
    p->ldy = ldy;
    p->bits = d->bits;
    return QP_OK;
}

qp_status qlinear_gemv(const qp_weight_desc *d, const qp_weight *w, const uint16_t *x, int64_t ldx, int64_t m,
                       uint16_t *y, int64_t ldy, void *stream)
{
    GemvProblem p;
    qp_status st = gemv_problem(d, w, x, ldx, m, y, ldy, &p);
    if (st != QP_OK) return st;
    return device(launch_gemv(p, S(stream)), "qlinear_gemv");
}

qp_status qlinear_gemv_batch(const qp_gemv_problem *problems, int32_t count, void *stream)
{
    if (!problems) return fail(QP_ERR_INVALID_ARG, "problems NULL");
    if (count < 1 || count > kMaxGemvBatch) return fail(QP_ERR_INVALID_ARG, "count=%d not in 1..%d", count, kMaxGemvBatch);
    GemvBatch b{};
    b.count = count;
    int64_t blocks = 0;
    int m_max = 1;
    for (int i = 0; i < count; ++i) {
        const qp_gemv_problem &q = problems[i];
        qp_status st = gemv_problem(&q.desc, &q.w, q.x, q.ldx, q.m, q.y, q.ldy, &b.p[i]);
        if (st != QP_OK) return st;
        if (b.p[i].gs != b.p[0].gs) return fail(QP_ERR_UNSUPPORTED, "one group size per batch");
        if (b.p[i].fp8 != b.p[0].fp8) return fail(QP_ERR_UNSUPPORTED, "fp16 and fp8 scales in one batch");
        if ((b.p[i].zrow != 0) != (b.p[0].zrow != 0))
            return fail(QP_ERR_UNSUPPORTED, "packed and byte zero points in one batch");
        b.p[i].block0 = blocks;
        blocks += q.desc.n / 16;
        if (q.m > m_max) m_max = (int)q.m;
    }
    if (blocks > 0x7FFFFFFF) return fail(QP_ERR_UNSUPPORTED, "too many row blocks");
    return device(launch_gemv_batch(b, blocks, m_max, S(stream)), "qlinear_gemv_batch");
}

// Workspace of qlinear_gemm: the outlier add-back's x^T and fp32 partial (nnz > 0), then the
// fp32 partials of a k-split GEMM (when its output tiles would leave most CUs idle).
static size_t gemm_outlier_bytes(const qp_weight_desc *d, int64_t m, int64_t nnz)
{
    if (nnz <= 0) return 0;
    const int64_t per = d->k * 2 + d->n * 4;  // n*k <= 2^40 keeps this far from overflow
    if (prod_over(per, gemm_xt_ld(m), 1, 1LL << 62)) return 0;
    return (size_t)(per * gemm_xt_ld(m));
}
static size_t gemm_split_bytes(const qp_weight_desc *d, int64_t m)
{
    const int s = gemm_split_parts(m, d->n, d->k);
    if (s < 2 || prod_over(m, d->n, 4 * s, 1LL << 40)) return 0;
    return (size_t)(4 * s * m * d->n);
}

size_t qlinear_gemm_workspace_bytes(const qp_weight_desc *d, int64_t m, int64_t nnz)
{
    if (check_desc(d, false) != QP_OK || m < 1 || m > (1LL << 24)) return 0;
    const size_t o = gemm_outlier_bytes(d, m, nnz);
    const size_t sp = gemm_split_bytes(d, m);
    return sp ? (o + 255) / 256 * 256 + sp : o;
}

qp_status qlinear_gemm(const qp_weight_desc *d, const qp_weight *w, const uint16_t *x, int64_t ldx, int64_t m,
                       uint16_t *y, int64_t ldy, void *workspace, size_t ws_bytes, void *stream)
{
    qp_status st = check_desc(d, true);
    if (st != QP_OK) return st;
    if ((st = check_weight(d, w, true)) != QP_OK) return st;
    if ((st = check_xy(d, x, ldx, m, y, ldy, d->n, 4)) != QP_OK) return st;
    if (m > (1LL << 24)) return fail(QP_ERR_INVALID_ARG, "m too large");
    if (prod_over(m, ldx, 2, 0x7FFFFFFFLL)) return fail(QP_ERR_UNSUPPORTED, "x larger than 2 GiB");
    if ((int64_t)qp_packed_bytes(d) > 0x7FFFFFFFLL) return fail(QP_ERR_UNSUPPORTED, "packed weight larger than 2 GiB");
    GemmArgs a{};
    a.ex[0] = weight_ptrs(d, w);
    a.fp8 = d->scale_format == QP_SCALE_FP8;  // check_weight has refused an outlier CSR with it
    a.zmid = zero_pair(d);
    a.gs = d->group_size;
    a.zrow = d->zero_mode == QP_ZERO_PACKED ? (uint32_t)zero_row_bytes(d) : 0u;
    const size_t need_o = gemm_outlier_bytes(d, m, w->nnz);
    if (w->nnz > 0) {
        if (prod_over(d->k, gemm_xt_ld(m), 2, 0x7FFFFFFFLL) || prod_over(d->n, gemm_xt_ld(m), 4, 0x7FFFFFFFLL))
            return fail(QP_ERR_UNSUPPORTED, "m*k or m*n too large for the outlier add-back");
        if (!workspace || ws_bytes < need_o || !aligned(workspace, 16))
            return fail(QP_ERR_WORKSPACE, "outlier add-back needs %zu bytes of workspace (16-byte aligned)", need_o);
        a.rowptr = w->csr_rowptr;
        a.col = w->csr_col;
        a.val = w->csr_val;
        a.ldxt = gemm_xt_ld(m);
        a.xt = (uint16_t *)workspace;
        a.spart = (float *)((uint8_t *)workspace + d->k * a.ldxt * 2);
    }
    // A workspace large enough for the k-split partials as well turns the split on (a shape
    // whose output tiles leave most CUs idle); without one the GEMM runs unsplit.
    const size_t need_s = gemm_split_bytes(d, m);
    const size_t off_s = (need_o + 255) / 256 * 256;
    if (need_s && workspace && aligned(workspace, 16) && ws_bytes >= off_s + need_s) {
        a.ksplit = gemm_split_parts(m, d->n, d->k);
        a.parts = (float *)((uint8_t *)workspace + off_s);
    }
    a.x = x;
    a.ldx = ldx;
    a.m = m;
    a.n = d->n;
    a.k = d->k;
    a.y = y;
    a.ldy = ldy;
    return device(launch_gemm(d->bits, a, S(stream)), "qlinear_gemm");
}

// The grouped launch after validation.  ksplit > 1 (fp32 rows only): k in ksplit equal parts,
// part p writing its partial rows at y + p * ysplit floats.
static qp_status grouped_launch(const qp_weight_desc *d, const qp_weight *experts, int32_t n_experts,
                                const uint16_t *x, int64_t ldx, const int32_t *row_src,
                                const int32_t *expert_offsets, int64_t rows, int32_t epilogue, void *y,
                                int64_t ldy, int32_t ksplit, int64_t ysplit, void *stream)
{
    // the launch's second grid dimension counts the occupied 32-row tiles (at most 65535)
    if ((rows + (int64_t)n_experts * 31) / 32 > 65535)
        return fail(QP_ERR_UNSUPPORTED, "grouped matmuls take at most 65535 32-row tiles of routed rows");
    GemmArgs a{};
    for (int e = 0; e < n_experts; ++e) a.ex[e] = weight_ptrs(d, &experts[e]);
    a.fp8 = d->scale_format == QP_SCALE_FP8;
    a.zmid = zero_pair(d);
    a.gs = d->group_size;
    a.zrow = d->zero_mode == QP_ZERO_PACKED ? (uint32_t)zero_row_bytes(d) : 0u;
    a.x = x;
    a.ldx = ldx;
    a.row_src = row_src;
    a.offsets = expert_offsets;
    a.m = rows;
    a.n = d->n;
    a.k = d->k;
    a.y = y;
    a.ldy = ldy;
    a.ksplit = ksplit;
    a.ysplit = ysplit;
    return device(launch_grouped(d->bits, epilogue, n_experts, a, S(stream)), "qlinear_grouped_gemm");
}

qp_status qlinear_grouped_gemm(const qp_weight_desc *d, const qp_weight *experts, int32_t n_experts,
                               const uint16_t *x, int64_t ldx, const int32_t *row_src,
                               const int32_t *expert_offsets, int64_t rows, int32_t epilogue, void *y,
                               int64_t ldy, void *stream)
{
    qp_status st = check_desc(d, true);
    if (st != QP_OK) return st;
    if (!experts) return fail(QP_ERR_INVALID_ARG, "experts NULL");
    if (n_experts < 1 || n_experts > kMaxExperts) return fail(QP_ERR_INVALID_ARG, "n_experts=%d not in 1..64", n_experts);
    for (int e = 0; e < n_experts; ++e)
        if ((st = check_weight(d, &experts[e], false)) != QP_OK) return st;
    if (epilogue != QP_EPI_NONE && epilogue != QP_EPI_SWIGLU && epilogue != QP_EPI_ROWS_F32)
        return fail(QP_ERR_INVALID_ARG, "epilogue=%d unknown", epilogue);
    if (epilogue == QP_EPI_SWIGLU && d->n % 32 != 0) return fail(QP_ERR_INVALID_ARG, "SwiGLU needs n %% 32 == 0");
    const int64_t ncols = epilogue == QP_EPI_SWIGLU ? d->n / 2 : d->n;
    if ((st = check_xy(d, x, ldx, rows < 1 ? 1 : rows, y, ldy, ncols, epilogue == QP_EPI_ROWS_F32 ? 8 : 4)) != QP_OK)
        return st;
    if (!expert_offsets) return fail(QP_ERR_INVALID_ARG, "expert_offsets NULL");
    if (rows < 0) return fail(QP_ERR_INVALID_ARG, "rows < 0");
    if (prod_over(rows, ldx, 2, 0x7FFFFFFFLL)) return fail(QP_ERR_UNSUPPORTED, "x larger than 2 GiB");
    if ((int64_t)qp_packed_bytes(d) > 0x7FFFFFFFLL) return fail(QP_ERR_UNSUPPORTED, "packed weight larger than 2 GiB");
    return grouped_launch(d, experts, n_experts, x, ldx, row_src, expert_offsets, rows, epilogue, y, ldy, 1, 0, stream);
}

qp_status qmoe_dispatch(const int32_t *ids, const float *w, int64_t tokens, int32_t topk, int32_t n_experts,
                        int32_t *offsets, int32_t *row_src, float *row_weight, int32_t *token_rows, void *stream)
{
    if (!ids || !w || !offsets || !row_src || !row_weight || !token_rows)
        return fail(QP_ERR_INVALID_ARG, "NULL pointer");
    if (tokens < 1 || topk < 1 || tokens * topk > 65536)
        return fail(QP_ERR_INVALID_ARG, "tokens*topk must be in 1..65536");
    if (n_experts < 1 || n_experts > kMaxExperts) return fail(QP_ERR_INVALID_ARG, "n_experts not in 1..64");
    return device(launch_moe_dispatch(ids, w, tokens, topk, n_experts, offsets, row_src, row_weight, token_rows,
                                      S(stream)),
                  "qmoe_dispatch");
}

qp_status qmoe_combine(const float *rows_f32, int64_t ld_rows, const int32_t *token_rows, const float *row_weight,
                       int64_t tokens, int32_t topk, int64_t n, uint16_t *out, int64_t ldo, void *stream)
{
    if (!rows_f32 || !token_rows || !row_weight || !out) return fail(QP_ERR_INVALID_ARG, "NULL pointer");
    if (tokens < 1 || topk < 1 || n < 1 || ld_rows < n || ldo < n)
        return fail(QP_ERR_INVALID_ARG, "bad sizes");
    if (tokens > 65535) return fail(QP_ERR_INVALID_ARG, "tokens > 65535");
    return device(launch_moe_combine(rows_f32, ld_rows, token_rows, row_weight, tokens, topk, n, out, ldo, 1, 0,
                                     S(stream)),
                  "qmoe_combine");
}

static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// The expert FFN computes the down projection in two k halves (each half a whole number of
// 512-k tile pairs): its grid then holds twice the workgroups of the one-pass launch, which
// fills the CUs' workgroup slots better; the halves' fp32 rows are summed by the combine.
static int32_t ffn_down_split(int64_t d_ff) { return d_ff % 512 == 0 ? 2 : 1; }

size_t qmoe_ffn_workspace_bytes(int64_t tokens, int32_t topk, int32_t n_experts, int64_t d_model, int64_t d_ff)
{
    if (tokens < 1 || topk < 1 || n_experts < 1 || d_model < 1 || d_ff < 1) return 0;
    const size_t R = (size_t)(tokens * topk);
    return al256((n_experts + 1) * 4) + 3 * al256(R * 4) + al256(R * (size_t)d_ff * 2) +
           ffn_down_split(d_ff) * al256(R * (size_t)d_model * 4);
}

qp_status qmoe_ffn(const qp_weight_desc *dgu, const qp_weight *gate_up, const qp_weight_desc *dd,
                   const qp_weight *down, int32_t n_experts, const uint16_t *x, int64_t ldx, int64_t tokens,
                   const int32_t *topk_ids, const float *topk_w, int32_t topk, uint16_t *out, int64_t ldo,
                   void *workspace, size_t ws_bytes, void *stream)
{
    qp_status st;
    if ((st = check_desc(dgu, true)) != QP_OK) return st;
    if ((st = check_desc(dd, true)) != QP_OK) return st;
    if (dgu->bits != dd->bits) return fail(QP_ERR_UNSUPPORTED, "gate/up and down must share the bit width");
    const int64_t d_model = dgu->k, d_ff = dgu->n / 2;
    if (dgu->n % 32 != 0 || dd->n != d_model || dd->k != d_ff)
        return fail(QP_ERR_INVALID_ARG, "shapes: gate_up must be [2*d_ff, d_model], down [d_model, d_ff]");
    if (d_ff % 8 != 0) return fail(QP_ERR_INVALID_ARG, "d_ff must be a multiple of 8");
    if (!out || !aligned(out, 2) || ldo < d_model) return fail(QP_ERR_INVALID_ARG, "out NULL/misaligned or ldo < d_model");
    const size_t need = qmoe_ffn_workspace_bytes(tokens, topk, n_experts, d_model, d_ff);
    if (!workspace || ws_bytes < need || !aligned(workspace, 256))
        return fail(QP_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned)", need);
    if (tokens < 1 || topk < 1 || tokens * topk > 65536) return fail(QP_ERR_INVALID_ARG, "tokens*topk must be in 1..65536");
    if (n_experts < 1 || n_experts > kMaxExperts) return fail(QP_ERR_INVALID_ARG, "n_experts not in 1..64");
    for (int e = 0; e < n_experts; ++e) {
        if ((st = check_weight(dgu, &gate_up[e], false)) != QP_OK) return st;
        if ((st = check_weight(dd, &down[e], false)) != QP_OK) return st;
    }
    if (!x || !aligned(x, 16) || ldx < d_model || ldx % 8 != 0) return fail(QP_ERR_INVALID_ARG, "x NULL/misaligned or bad ldx");
    if (!topk_ids || !topk_w) return fail(QP_ERR_INVALID_ARG, "routing NULL");
    // The down projection reads the fp16 intermediate [tokens*topk][d_ff] through one buffer
    // resource, as qlinear_grouped_gemm reads x: it must stay within 2 GiB.
    if (tokens * topk * d_ff * 2 > 0x7FFFFFFFLL)
        return fail(QP_ERR_UNSUPPORTED, "tokens*topk*d_ff*2 = %lld bytes of intermediate exceed 2 GiB",
                    (long long)(tokens * topk * d_ff * 2));
    if (prod_over(tokens, ldx, 2, 0x7FFFFFFFLL)) return fail(QP_ERR_UNSUPPORTED, "x larger than 2 GiB");

    const size_t R = (size_t)(tokens * topk);
    uint8_t *p = (uint8_t *)workspace;
    int32_t *offsets = (int32_t *)p;
    p += al256((n_experts + 1) * 4);
    int32_t *row_src = (int32_t *)p;
    p += al256(R * 4);
    float *row_weight = (float *)p;
    p += al256(R * 4);
    int32_t *token_rows = (int32_t *)p;
    p += al256(R * 4);
    uint16_t *act = (uint16_t *)p;
    p += al256(R * (size_t)d_ff * 2);
    float *rows = (float *)p;

    if ((st = qmoe_dispatch(topk_ids, topk_w, tokens, topk, n_experts, offsets, row_src, row_weight, token_rows,
                            stream)) != QP_OK)
        return st;
    if ((st = qlinear_grouped_gemm(dgu, gate_up, n_experts, x, ldx, row_src, offsets, (int64_t)R, QP_EPI_SWIGLU,
                                   act, d_ff, stream)) != QP_OK)
        return st;
    const int32_t ks = ffn_down_split(d_ff);
    const int64_t ystride = (int64_t)(al256(R * (size_t)d_model * 4) / 4);
    if ((st = grouped_launch(dd, down, n_experts, act, d_ff, nullptr, offsets, (int64_t)R, QP_EPI_ROWS_F32, rows,
                             d_model, ks, ystride, stream)) != QP_OK)
        return st;
    return device(launch_moe_combine(rows, d_model, token_rows, row_weight, tokens, topk, d_model, out, ldo, ks,
                                     ystride, S(stream)),
                  "qmoe_combine");
}

size_t qkv_cache_bytes(const qkv_desc *d, int32_t which)
{
    if (check_kv(d) != QP_OK || (which != QKV_K && which != QKV_V)) return 0;
    return (size_t)kv_rows(d) * 128 * (which == QKV_K ? d->k_bits : d->v_bits) / 8;
}

size_t qkv_scale_count(const qkv_desc *d, int32_t which)
{
    if (check_kv(d) != QP_OK || (which != QKV_K && which != QKV_V)) return 0;
    return (size_t)kv_rows(d) * (128 / (which == QKV_K ? d->k_group : d->v_group));
}

qp_status qkv_quantize(const qkv_desc *d, int32_t which, const uint16_t *x, int64_t ldx, const int64_t *slots,
                       int64_t rows, void *codes, float *scales, void *stream)
{
    qp_status st;
    if ((st = check_kv(d)) != QP_OK) return st;
    if (which != QKV_K && which != QKV_V) return fail(QP_ERR_INVALID_ARG, "which=%d (QKV_K or QKV_V)", which);
    if (rows < 0) return fail(QP_ERR_INVALID_ARG, "rows < 0");
    if (rows > 0 && (!x || !aligned(x, 16) || ldx < 128 || ldx % 8 != 0))
        return fail(QP_ERR_INVALID_ARG, "x NULL/misaligned or bad ldx");
    if (rows > 0 && !slots) return fail(QP_ERR_INVALID_ARG, "slots NULL");
    if (!codes || !aligned(codes, 16) || !scales || !aligned(scales, 16))
        return fail(QP_ERR_INVALID_ARG, "codes/scales NULL or not 16-byte aligned");
    if (rows > (1LL << 31) - 4) return fail(QP_ERR_INVALID_ARG, "too many rows");
    KvQuantArgs a{};
    a.x = x;
    a.ldx = ldx;
    a.slots = slots;
    a.rows = rows;
    a.total_rows = kv_rows(d);
    a.cap = d->capacity;
    a.codes = (uint8_t *)codes;
    a.scales = scales;
    const int bits = which == QKV_K ? d->k_bits : d->v_bits, g = which == QKV_K ? d->k_group : d->v_group;
    return device(launch_kv_quantize(bits, which, g, a, S(stream)), "kv quantize");
}

size_t qattn_decode_workspace_bytes(const qkv_desc *d)
{
    if (check_kv(d) != QP_OK) return 0;
    int32_t ns, ch;
    kv_split(d->batch, d->kv_heads, d->capacity, &ns, &ch);
    if (ns == 1) return 0;
    const size_t parts = (size_t)d->batch * d->q_heads * ns;
    return parts * 128 * 4 + parts * 2 * 4;
}

qp_status qattn_decode(const qkv_desc *d, const uint16_t *q, const void *k_codes, const float *k_scales,
                       const void *v_codes, const float *v_scales, const int32_t *seq_lens, float sm_scale,
                       uint16_t *o, void *workspace, size_t ws_bytes, void *stream)
{
    qp_status st;
    if ((st = check_kv(d)) != QP_OK) return st;
    if (!q || !aligned(q, 16) || !o || !aligned(o, 16)) return fail(QP_ERR_INVALID_ARG, "q/o NULL or not 16-byte aligned");
    if (!k_codes || !aligned(k_codes, 16) || !v_codes || !aligned(v_codes, 16) || !k_scales ||
        !aligned(k_scales, 16) || !v_scales || !aligned(v_scales, 16))
        return fail(QP_ERR_INVALID_ARG, "cache codes/scales NULL or not 16-byte aligned");
    if (!seq_lens) return fail(QP_ERR_INVALID_ARG, "seq_lens NULL");
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
        return fail(QP_ERR_INVALID_ARG, "sm_scale not finite");
    const size_t need = qattn_decode_workspace_bytes(d);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16)))
        return fail(QP_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned)", need);
    KvAttnArgs a{};
    a.q = q;
    a.kc = (const uint8_t *)k_codes;
    a.ks = k_scales;
    a.vc = (const uint8_t *)v_codes;
    a.vs = v_scales;
    a.lens = seq_lens;
    a.o = o;
    a.cap = d->capacity;
    a.hq = d->q_heads;
    a.hkv = d->kv_heads;
    a.grp = d->q_heads / d->kv_heads;
    kv_split(d->batch, d->kv_heads, d->capacity, &a.nsplit, &a.chunk);
    if (a.nsplit > 1) {
        const size_t parts = (size_t)d->batch * d->q_heads * a.nsplit;
        a.part_o = (float *)workspace;
        a.part_ml = (float *)((uint8_t *)workspace + parts * 128 * 4);
    }
    a.c = (float)((double)sm_scale * 1.4426950408889634);
    return device(launch_kv_attn(d->k_bits, d->v_bits, d->k_group, d->v_group, d->batch, a, S(stream)),
                  "kv attention");
}

qp_status qattn_decode_noalloc(const qkv_desc *d, const uint16_t *q, const void *k_codes, const float *k_scales,
                               const void *v_codes, const float *v_scales, const int32_t *seq_lens, float sm_scale,
                               uint16_t *o, void *stream)
{
    qp_status st;
    if ((st = check_kv(d)) != QP_OK) return st;
    const size_t need = qattn_decode_workspace_bytes(d);
    if (need > QATTN_NOALLOC_SCRATCH_BYTES)
        return fail(QP_ERR_WORKSPACE,
                    "qattn_decode_noalloc: this shape needs %zu bytes of scratch, above its fixed %u bytes; "
                    "use qattn_decode with a workspace",
                    need, (unsigned)QATTN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != QP_OK) return st;
    return qattn_decode(d, q, k_codes, k_scales, v_codes, v_scales, seq_lens, sm_scale, o, ws, need, stream);
}

qp_status qact_quantize(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int8_t *xq, float *x_scales,
                        void *stream)
{
    if (!x || !aligned(x, 16)) return fail(QP_ERR_INVALID_ARG, "x NULL or not 16-byte aligned");
    if (!xq || !aligned(xq, 8)) return fail(QP_ERR_INVALID_ARG, "xq NULL or not 8-byte aligned");
    if (!x_scales || !aligned(x_scales, 4)) return fail(QP_ERR_INVALID_ARG, "x_scales NULL or misaligned");
    if (k <= 0 || k % kGroup != 0) return fail(QP_ERR_INVALID_ARG, "k=%lld must be a positive multiple of 128", (long long)k);
    if (ldx < k || ldx % 8 != 0) return fail(QP_ERR_INVALID_ARG, "ldx=%lld must be >= k and a multiple of 8", (long long)ldx);
    if (m < 1 || m > 0x7FFFFFFFLL) return fail(QP_ERR_INVALID_ARG, "m=%lld not in 1..2^31-1", (long long)m);
    if (prod_over(m, ldx, 2, 1LL << 62) || prod_over(m, k, 1, 1LL << 62)) return fail(QP_ERR_INVALID_ARG, "x or xq too large");
    return device(launch_act_quantize(x, ldx, m, k, xq, x_scales, S(stream)), "qact_quantize");
}

qp_status qlinear_gemm_a8(const qp_weight_desc *d, const qp_weight *w, const int8_t *xq, const float *x_scales,
                          int64_t m, uint16_t *y, int64_t ldy, void *stream)
{
    qp_status st = check_desc(d, true);
    if (st != QP_OK) return st;
    if (d->group_size != kGroup) return fail(QP_ERR_UNSUPPORTED, "the int8 GEMM is built for groups of 128");
    if ((st = check_weight(d, w, false)) != QP_OK) return st;
    if (w->nnz > 0) return fail(QP_ERR_UNSUPPORTED, "outliers are not applied on int8 activations");
    if (!xq || !aligned(xq, 16)) return fail(QP_ERR_INVALID_ARG, "xq NULL or not 16-byte aligned");
    if (!x_scales || !aligned(x_scales, 4)) return fail(QP_ERR_INVALID_ARG, "x_scales NULL or misaligned");
    if (!y || !aligned(y, 8)) return fail(QP_ERR_INVALID_ARG, "y NULL or misaligned");
    if (ldy < d->n || ldy % 4 != 0) return fail(QP_ERR_INVALID_ARG, "ldy=%lld must be >= %lld and a multiple of 4", (long long)ldy, (long long)d->n);
    if (m < 1) return fail(QP_ERR_INVALID_ARG, "m=%lld must be >= 1", (long long)m);
    if (prod_over(m, d->k, 1, 0x7FFFFFFFLL)) return fail(QP_ERR_UNSUPPORTED, "xq larger than 2 GiB");
    if ((int64_t)qp_packed_bytes(d) > 0x7FFFFFFFLL) return fail(QP_ERR_UNSUPPORTED, "packed weight larger than 2 GiB");
    const ExpertPtrs ep = weight_ptrs(d, w);
    const uint32_t zrow = d->zero_mode == QP_ZERO_PACKED ? (uint32_t)zero_row_bytes(d) : 0u;
    return device(launch_gemm_a8(d->bits, ep, d->scale_format == QP_SCALE_FP8, xq, x_scales, m, d->n, d->k, zero_pair(d),
                                 zrow, y, ldy, S(stream)),
                  "qlinear_gemm_a8");
}

}  // extern "C"
