// Serialized packed-weight blob: a quantized, packed weight (codes, scales, zero points and
// the outlier CSR) as one self-describing byte string for storing and reloading without
// repacking (the one-time repack of the single-GPU 70B page, s3).  Every field and array
// element is written byte by byte in little-endian order, so the bytes do not depend on the
// host's byte order (the mixed-bit page, s3.2, reads units as little-endian integers and warns
// that endianness must be fixed).  Host code only: blobs live in host memory.
//
// Layout (offsets in bytes):
//   0  magic "QPKW"            4  u32 version (1)         8  u32 header bytes (64)
//  12  i32 bits               16  i32 group size          20  i32 layout
//  24  i32 zero mode          28  u32 flags (0)           32  i64 n
//  40  i64 k                  48  i64 nnz                 56  u32 CRC-32 of the blob (this
//                                                             field counted as zeros)
//  60  u32 reserved (0)
//  64  sections, each starting at a multiple of 64: packed codes (u8), scales (u16 each),
//      zero points (u8; absent for implied zero points), and when nnz > 0 the CSR row
//      pointers (i32, n + 1), columns (i32, nnz) and values (u16, nnz).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "qpack.h"

namespace qp {
qp_status fail(qp_status st, const char *fmt, ...);
}

namespace {

constexpr uint32_t kVersion = 1;
constexpr uint32_t kHeader = 64;

size_t al64(size_t v) { return (v + 63) & ~(size_t)63; }

// CRC-32 (IEEE 802.3 polynomial, reflected 0xEDB88320, initial and final value 0xFFFFFFFF):
// the byte table is the bitwise definition applied to each byte value.
struct CrcTable {
    uint32_t t[256];
    CrcTable()
    {
        for (uint32_t v = 0; v < 256; ++v) {
            uint32_t c = v;
            for (int b = 0; b < 8; ++b) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
            t[v] = c;
        }
    }
};

uint32_t crc_run(uint32_t c, const uint8_t *p, size_t n)
{
    static const CrcTable tab;
    for (size_t i = 0; i < n; ++i) c = tab.t[(c ^ p[i]) & 0xFF] ^ (c >> 8);
    return c;
}

// CRC-32 of the whole blob with its checksum field (bytes 56..59) counted as zeros.
uint32_t blob_crc(const uint8_t *b, size_t total)
{
    uint8_t head[64];
    memcpy(head, b, 64);
    memset(head + 56, 0, 4);
    const uint32_t c = crc_run(0xFFFFFFFFu, head, 64);
    return crc_run(c, b + 64, total - 64) ^ 0xFFFFFFFFu;
}

void put_u32(uint8_t *p, uint32_t v)
{
    for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
void put_u64(uint8_t *p, uint64_t v)
{
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
uint32_t get_u32(const uint8_t *p)
{
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
    return v;
}
uint64_t get_u64(const uint8_t *p)
{
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
    return v;
}

struct Sections {
    size_t packed, scales, zeros, rowptr, col, val;  // offsets
    size_t n_packed, n_scales, n_zeros, n_rowptr, n_col, n_val;  // byte sizes
    size_t total;
};

// Section sizes and offsets, or false if the descriptor is not a valid weight.
bool sections(const qp_weight_desc *d, int64_t nnz, Sections *s)
{
    if (nnz < 0 || d->scale_format != QP_SCALE_FP16) return false;
    const size_t pb = qp_packed_bytes(d);
    if (pb == 0 || nnz > d->n * d->k) return false;  // a valid desc keeps n*k <= 2^40: no overflow below
    s->n_packed = pb;
    s->n_scales = qp_num_groups(d) * 2;
    s->n_zeros = qp_zero_bytes(d);
    s->n_rowptr = nnz > 0 ? (size_t)(d->n + 1) * 4 : 0;
    s->n_col = (size_t)nnz * 4;
    s->n_val = (size_t)nnz * 2;
    size_t o = kHeader;
    s->packed = o;
    o = al64(o + s->n_packed);
    s->scales = o;
    o = al64(o + s->n_scales);
    s->zeros = o;
    o = al64(o + s->n_zeros);
    s->rowptr = o;
    o = al64(o + s->n_rowptr);
    s->col = o;
    o = al64(o + s->n_col);
    s->val = o;
    o = al64(o + s->n_val);
    s->total = o;
    return true;
}

}  // namespace

extern "C" {

size_t qp_blob_bytes(const qp_weight_desc *d, int64_t nnz)
{
    Sections s;
    return d && sections(d, nnz, &s) ? s.total : 0;
}

qp_status qp_blob_write(const qp_weight_desc *d, const qp_weight *w, void *blob, size_t blob_bytes)
{
    if (!d || !w || !blob) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_write: NULL argument");
    Sections s;
    if (d->scale_format != QP_SCALE_FP16) return qp::fail(QP_ERR_UNSUPPORTED, "qp_blob_write: the blob holds fp16 scales");
    if (!sections(d, w->nnz, &s)) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_write: invalid descriptor or nnz");
    if (blob_bytes < s.total)
        return qp::fail(QP_ERR_WORKSPACE, "qp_blob_write: blob needs %zu bytes, got %zu", s.total, blob_bytes);
    if (!w->packed || !w->scales || (s.n_zeros && !w->zeros))
        return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_write: packed/scales/zeros NULL");
    if (w->nnz > 0 && (!w->csr_rowptr || !w->csr_col || !w->csr_val))
        return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_write: CSR arrays NULL with nnz > 0");
    uint8_t *b = (uint8_t *)blob;
    memset(b, 0, s.total);
    memcpy(b, "QPKW", 4);
    put_u32(b + 4, kVersion);
    put_u32(b + 8, kHeader);
    put_u32(b + 12, (uint32_t)d->bits);
    put_u32(b + 16, (uint32_t)d->group_size);
    put_u32(b + 20, (uint32_t)d->layout);
    put_u32(b + 24, (uint32_t)d->zero_mode);
    put_u64(b + 32, (uint64_t)d->n);
    put_u64(b + 40, (uint64_t)d->k);
    put_u64(b + 48, (uint64_t)w->nnz);
    memcpy(b + s.packed, w->packed, s.n_packed);
    for (size_t i = 0; i < s.n_scales / 2; ++i) {
        const uint16_t v = w->scales[i];
        b[s.scales + 2 * i] = (uint8_t)v;
        b[s.scales + 2 * i + 1] = (uint8_t)(v >> 8);
    }
    if (s.n_zeros) memcpy(b + s.zeros, w->zeros, s.n_zeros);
    if (w->nnz > 0) {
        for (int64_t i = 0; i <= d->n; ++i) put_u32(b + s.rowptr + 4 * i, (uint32_t)w->csr_rowptr[i]);
        for (int64_t i = 0; i < w->nnz; ++i) {
            put_u32(b + s.col + 4 * i, (uint32_t)w->csr_col[i]);
            b[s.val + 2 * i] = (uint8_t)w->csr_val[i];
            b[s.val + 2 * i + 1] = (uint8_t)(w->csr_val[i] >> 8);
        }
    }
    put_u32(b + 56, blob_crc(b, s.total));
    return QP_OK;
}

qp_status qp_blob_parse(const void *blob, size_t blob_bytes, qp_weight_desc *desc_out, int64_t *nnz_out,
                        size_t *offsets_out)
{
    if (!blob || !desc_out || !nnz_out) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: NULL argument");
    const uint8_t *b = (const uint8_t *)blob;
    if (blob_bytes < kHeader) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: %zu bytes, shorter than the header", blob_bytes);
    if (memcmp(b, "QPKW", 4) != 0) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: bad magic");
    if (get_u32(b + 4) != kVersion)
        return qp::fail(QP_ERR_UNSUPPORTED, "qp_blob_parse: version %u (only %u is known)", get_u32(b + 4), kVersion);
    if (get_u32(b + 8) != kHeader || get_u32(b + 28) != 0 || get_u32(b + 60) != 0)
        return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: bad header size or reserved fields");
    qp_weight_desc d{};
    d.bits = (int32_t)get_u32(b + 12);
    d.group_size = (int32_t)get_u32(b + 16);
    d.layout = (int32_t)get_u32(b + 20);
    d.zero_mode = (int32_t)get_u32(b + 24);
    d.n = (int64_t)get_u64(b + 32);
    d.k = (int64_t)get_u64(b + 40);
    const int64_t nnz = (int64_t)get_u64(b + 48);
    Sections s;
    if (!sections(&d, nnz, &s)) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: invalid weight description");
    if (blob_bytes < s.total)
        return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: truncated (%zu of %zu bytes)", blob_bytes, s.total);
    if (blob_crc(b, s.total) != get_u32(b + 56))
        return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: checksum mismatch");
    if (nnz > 0) {  // CSR consistency: rowptr starts at 0, never decreases, ends at nnz; columns in range
        int64_t prev = 0;
        for (int64_t i = 0; i <= d.n; ++i) {
            const int64_t v = (int32_t)get_u32(b + s.rowptr + 4 * i);
            if ((i == 0 && v != 0) || v < prev || v > nnz) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: bad CSR row pointers");
            prev = v;
        }
        if (prev != nnz) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: CSR row pointers end at %lld, nnz %lld", (long long)prev, (long long)nnz);
        for (int64_t i = 0; i < nnz; ++i) {
            const int64_t c = (int32_t)get_u32(b + s.col + 4 * i);
            if (c < 0 || c >= d.k) return qp::fail(QP_ERR_INVALID_ARG, "qp_blob_parse: CSR column out of range");
        }
    }
    *desc_out = d;
    *nnz_out = nnz;
    if (offsets_out) {
        offsets_out[0] = s.packed;
        offsets_out[1] = s.scales;
        offsets_out[2] = s.n_zeros ? s.zeros : 0;
        offsets_out[3] = nnz > 0 ? s.rowptr : 0;
        offsets_out[4] = nnz > 0 ? s.col : 0;
        offsets_out[5] = nnz > 0 ? s.val : 0;
    }
    return QP_OK;
}

}  // extern "C"
