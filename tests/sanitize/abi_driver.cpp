// Host sanitizer driver for the C ABI's host code: argument validation of every entry point
// (each call fails validation before anything is launched, so no GPU is touched) and the
// packed-weight blob parser under random corruption.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side by tests/test_sanitize.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "qpack.h"

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

static uint64_t g_s = 0x243F6A8885A308D3ull;
static uint32_t rnd()
{
    g_s ^= g_s << 13;
    g_s ^= g_s >> 7;
    g_s ^= g_s << 17;
    return (uint32_t)(g_s >> 32);
}

static qp_weight_desc desc(int bits, int64_t n, int64_t k, int layout = QP_LAYOUT_DEVICE, int g = 128, int zm = 0)
{
    qp_weight_desc d{};
    d.bits = bits;
    d.group_size = g;
    d.layout = layout;
    d.zero_mode = zm;
    d.n = n;
    d.k = k;
    return d;
}

int main()
{
    void *F = (void *)0x10000;  // aligned, never dereferenced
    const uint16_t *FH = (const uint16_t *)F;
    // byte accounting at the edges
    for (int bits = -1; bits <= 9; ++bits)
        for (int64_t k : {0LL, 128LL, 256LL, 300LL, 1LL << 30})
            (void)qp_packed_bytes(&(const qp_weight_desc &)desc(bits, 16, k));
    CHECK(qp_packed_bytes(nullptr) == 0);
    CHECK(qp_outlier_count(-1, 5, 0.1) == 0);
    qp_weight_desc big = desc(4, 1LL << 40, 1LL << 20);
    CHECK(qp_packed_bytes(&big) == 0);
    // validation failures of the entry points
    qp_weight_desc d = desc(4, 256, 512);
    qp_weight w = {F, FH, (const uint8_t *)F, nullptr, nullptr, nullptr, 0};
    int64_t nnz = 0;
    CHECK(qpack_quantize(&d, nullptr, 512, 0.0, (uint8_t *)F, (uint16_t *)F, (uint8_t *)F, nullptr, nullptr,
                         nullptr, 0, &nnz, nullptr, 0, nullptr) == QP_ERR_INVALID_ARG);
    CHECK(qpack_quantize(&d, FH, 512, 0.5, (uint8_t *)F, (uint16_t *)F, (uint8_t *)F, (int32_t *)F, (int32_t *)F,
                         (uint16_t *)F, 3, &nnz, nullptr, 0, nullptr) == QP_ERR_WORKSPACE);
    CHECK(qpack_pack(&d, (const uint8_t *)F, (void *)0x10001, nullptr) == QP_ERR_INVALID_ARG);
    CHECK(qlinear_gemv(&d, &w, FH, 512, 17, (uint16_t *)F, 256, nullptr) == QP_ERR_UNSUPPORTED);
    CHECK(qlinear_gemv(&d, &w, FH, 500, 1, (uint16_t *)F, 256, nullptr) == QP_ERR_INVALID_ARG);
    qp_weight wc = w;
    wc.nnz = 5;
    CHECK(qlinear_gemv(&d, &wc, FH, 512, 1, (uint16_t *)F, 256, nullptr) == QP_ERR_INVALID_ARG);
    CHECK(qlinear_gemm(&d, &w, FH, 512, 0, (uint16_t *)F, 256, nullptr, 0, nullptr) == QP_ERR_INVALID_ARG);
    qp_gemv_problem probs[9];
    CHECK(qlinear_gemv_batch(probs, 9, nullptr) == QP_ERR_INVALID_ARG);
    CHECK(qlinear_gemv_batch(nullptr, 1, nullptr) == QP_ERR_INVALID_ARG);
    std::vector<qp_weight> ex(65, w);
    CHECK(qlinear_grouped_gemm(&d, ex.data(), 65, FH, 512, (const int32_t *)F, (const int32_t *)F, 10, 0,
                               (void *)F, 256, nullptr) == QP_ERR_INVALID_ARG);
    CHECK(qmoe_dispatch((const int32_t *)F, (const float *)F, 40000, 2, 16, (int32_t *)F, (int32_t *)F, (float *)F,
                        (int32_t *)F, nullptr) == QP_ERR_INVALID_ARG);
    qp_weight_desc gu = desc(4, 2 * 16384, 4096), dn = desc(4, 4096, 16384);
    std::vector<qp_weight> e16(16, w);
    const size_t need = qmoe_ffn_workspace_bytes(32768, 2, 16, 4096, 16384);
    CHECK(qmoe_ffn(&gu, e16.data(), &dn, e16.data(), 16, FH, 4096, 32768, (const int32_t *)F, (const float *)F, 2,
                   (uint16_t *)F, 4096, F, need, nullptr) == QP_ERR_UNSUPPORTED);
    qkv_desc kd = {1, 256, 16, 128, 4, 8, 64, 64, 32768};
    CHECK(qattn_decode_noalloc(&kd, FH, F, (const float *)F, F, (const float *)F, (const int32_t *)F, 0.1f,
                               (uint16_t *)F, nullptr) == QP_ERR_WORKSPACE);
    kd.q_heads = 300;
    CHECK(qattn_decode(&kd, FH, F, (const float *)F, F, (const float *)F, (const int32_t *)F, 0.1f, (uint16_t *)F,
                       nullptr, 0, nullptr) != QP_OK);
    CHECK(strlen(qp_last_error()) > 0);
    // sizes whose products overflow 64 bits are refused, not wrapped
    qp_weight_desc huge = desc(4, 16, 1LL << 62);
    CHECK(qlinear_gemv(&huge, &w, FH, 1LL << 62, 1, (uint16_t *)F, 16, nullptr) != QP_OK);
    CHECK(qlinear_gemv(&d, &w, FH, 1LL << 61, 16, (uint16_t *)F, 256, nullptr) == QP_ERR_UNSUPPORTED);
    CHECK(qlinear_gemm(&d, &w, FH, 1LL << 61, 1000, (uint16_t *)F, 256, nullptr, 0, nullptr) == QP_ERR_UNSUPPORTED);
    CHECK(qlinear_gemm_workspace_bytes(&d, 1LL << 40, 5) == 0);
    CHECK(qlinear_grouped_gemm(&d, ex.data(), 1, FH, 1LL << 61, (const int32_t *)F, (const int32_t *)F, 100, 0,
                               (void *)F, 256, nullptr) == QP_ERR_UNSUPPORTED);

    // blob: a valid blob from synthetic host arrays, then random corruption
    const int64_t n = 32, k = 512, G = k / 128, bnnz = 7;
    qp_weight_desc bd = desc(5, n, k);
    std::vector<uint8_t> packed(n * k * 5 / 8), zeros(n * G);
    std::vector<uint16_t> scales(n * G), val(bnnz);
    std::vector<int32_t> rowptr(n + 1), col(bnnz);
    for (auto &v : packed) v = (uint8_t)rnd();
    for (auto &v : scales) v = (uint16_t)rnd();
    for (auto &v : zeros) v = (uint8_t)(rnd() & 31);
    for (int64_t i = 0; i <= n; ++i) rowptr[i] = (int32_t)(i * bnnz / n);
    for (int64_t i = 0; i < bnnz; ++i) {
        col[i] = (int32_t)(rnd() % k);
        val[i] = (uint16_t)rnd();
    }
    qp_weight bw = {packed.data(), scales.data(), zeros.data(), rowptr.data(), col.data(), val.data(), bnnz};
    const size_t bb = qp_blob_bytes(&bd, bnnz);
    std::vector<uint8_t> blob(bb);
    CHECK(qp_blob_write(&bd, &bw, blob.data(), bb) == QP_OK);
    qp_weight_desc od;
    int64_t onnz = 0;
    size_t offs[6];
    CHECK(qp_blob_parse(blob.data(), bb, &od, &onnz, offs) == QP_OK && onnz == bnnz);
    int ok = 0;
    for (int it = 0; it < 30000; ++it) {
        std::vector<uint8_t> b = blob;
        const int muts = 1 + (int)(rnd() % 4);
        for (int m = 0; m < muts; ++m) {
            const size_t pos = rnd() % (rnd() % 2 ? 64 : b.size());  // header bytes half the time
            b[pos] = (uint8_t)rnd();
        }
        size_t len = b.size();
        if (rnd() % 8 == 0) len = rnd() % (b.size() + 1);
        // a heap copy of exactly `len` bytes, so reads past the end are caught
        uint8_t *h = (uint8_t *)malloc(len ? len : 1);
        memcpy(h, b.data(), len);
        if (qp_blob_parse(h, len, &od, &onnz, offs) == QP_OK) ++ok;
        free(h);
    }
    printf("abi driver ok (%d corrupted blobs accepted: mutations that kept the checksum)\n", ok);
    return 0;
}
