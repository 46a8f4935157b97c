/* Host sanitizer driver for the CPU oracle (oracle/qoracle.c): every routine on small inputs
 * and on the edge cases the tests pin (all-zero and subnormal groups, outliers with ties, every
 * bit width and layout, ragged and empty decode lengths, lengths above the cache capacity).
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py; any
 * report aborts the run.  Round trips are checked so the inputs exercise the real paths. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double or_half_value(uint16_t h);
uint16_t or_round_half(double x);
void or_quantize_group(const uint16_t *w, int n, int bits, uint16_t *s, uint8_t *z, uint8_t *q);
void or_quantize_group_sym(const uint16_t *w, int n, int bits, uint16_t *s, uint8_t *q);
int or_quantize(int64_t N, int64_t K, int bits, int g, int zero_mode, const uint16_t *w, int64_t ldw,
                double frac, uint8_t *codes, uint16_t *scales, uint8_t *zeros, int32_t *rowptr, int32_t *col,
                uint16_t *val, int64_t cap, int64_t *nnz_out);
void or_pack_canonical(int64_t N, int64_t K, int bits, const uint8_t *codes, uint8_t *out);
void or_unpack_canonical(int64_t N, int64_t K, int bits, const uint8_t *in, uint8_t *codes);
int or_pack_device(int64_t N, int64_t K, int bits, const uint8_t *codes, uint8_t *out);
int or_unpack_device(int64_t N, int64_t K, int bits, const uint8_t *in, uint8_t *codes);
void or_linear(int64_t M, int64_t N, int64_t K, int g, const uint16_t *x, int64_t ldx, const uint8_t *codes,
               const uint16_t *scales, const uint8_t *zeros, const int32_t *rowptr, const int32_t *col,
               const uint16_t *val, double *r, int64_t ldr);
void or_moe_ffn(int64_t T, int64_t D, int64_t F, int topk, int g, const int32_t *ids, const float *wts,
                const uint16_t *x, const uint8_t *gc, const uint16_t *gs, const uint8_t *gz, const uint8_t *uc,
                const uint16_t *us, const uint8_t *uz, const uint8_t *dc, const uint16_t *ds, const uint8_t *dz,
                double *r);
int64_t or_zero_row_bytes(int64_t G, int bits);
void or_pack_zeros(int64_t N, int64_t G, int bits, const uint8_t *zeros, uint8_t *out);
void or_unpack_zeros(int64_t N, int64_t G, int bits, const uint8_t *in, uint8_t *zeros);
void or_kv_quantize_rows(const uint16_t *x, int64_t rows, int g, int bits, uint8_t *codes, float *scales);
void or_kv_layout(int which, int bits, int64_t cap, int64_t rows, const int64_t *slot, const uint8_t *codes,
                  uint8_t *cache);
void or_kv_unlayout(int which, int bits, int64_t cap, int64_t rows, const int64_t *slot, const uint8_t *cache,
                    uint8_t *codes);
void or_attn_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t cap, int kbits, int kg, int vbits, int vg,
                    const uint16_t *q, const uint8_t *kc, const float *ks, const uint8_t *vc, const float *vs,
                    const int32_t *len, double sm_scale, double *o, double *a);

static uint64_t g_s = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    g_s ^= g_s << 13;
    g_s ^= g_s >> 7;
    g_s ^= g_s << 17;
    return (double)(g_s >> 11) / 9007199254740992.0;
}
static uint16_t hrand(double scale) { return or_round_half((urand() * 2.0 - 1.0) * scale); }

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void)
{
    for (uint32_t h = 0; h < 65536; ++h)
        if ((h & 0x7C00) != 0x7C00) CHECK(or_round_half(or_half_value((uint16_t)h)) == h || (h == 0x8000));

    uint16_t grp[128], sc;
    uint8_t zp, q[128];
    for (int bits = 2; bits <= 6; ++bits)
        for (int gsz = 32; gsz <= 128; gsz *= 2) {
            memset(grp, 0, sizeof grp);
            or_quantize_group(grp, gsz, bits, &sc, &zp, q);
            grp[3] = 1; /* smallest subnormal */
            or_quantize_group(grp, gsz, bits, &sc, &zp, q);
            or_quantize_group_sym(grp, gsz, bits, &sc, q);
            for (int i = 0; i < gsz; ++i) grp[i] = hrand(0.05);
            or_quantize_group(grp, gsz, bits, &sc, &zp, q);
            or_quantize_group_sym(grp, gsz, bits, &sc, q);
        }

    enum { N = 16, K = 512, M = 3 };
    uint16_t *w = malloc(sizeof(uint16_t) * N * K), *x = malloc(sizeof(uint16_t) * M * K);
    for (int i = 0; i < N * K; ++i) w[i] = hrand(0.05);
    for (int i = 0; i < 40; ++i) w[(i * 197) % (N * K)] = or_round_half(i % 2 ? 4.0 : -4.0); /* ties */
    for (int i = 0; i < M * K; ++i) x[i] = hrand(2.0);
    uint8_t *codes = malloc(N * K), *codes2 = malloc(N * K), *packed = malloc(N * K);
    uint16_t *scales = malloc(sizeof(uint16_t) * N * (K / 32));
    uint8_t *zeros = malloc(N * (K / 32)), *zeros2 = malloc(N * (K / 32));
    uint8_t *pz = malloc((size_t)N * or_zero_row_bytes(K / 32, 6));
    int32_t rowptr[N + 1], col[64];
    uint16_t val[64];
    double *r = malloc(sizeof(double) * M * N);
    int64_t nnz = 0;
    CHECK(or_quantize(N, K, 4, 128, 0, w, K, 30.0 / (N * K), codes, scales, zeros, rowptr, col, val, 10, &nnz) == 1);
    for (int bits = 2; bits <= 6; ++bits)
        for (int g = 32; g <= 128; g *= 2)
            for (int zm = 0; zm <= 1; ++zm) {
                CHECK(or_quantize(N, K, bits, g, zm, w, K, 30.0 / (N * K), codes, scales, zm ? NULL : zeros, rowptr,
                                  col, val, 64, &nnz) == 0);
                CHECK(nnz == 30);
                or_pack_canonical(N, K, bits, codes, packed);
                or_unpack_canonical(N, K, bits, packed, codes2);
                CHECK(memcmp(codes, codes2, N * K) == 0);
                CHECK(or_pack_device(N, K, bits, codes, packed) == 0);
                CHECK(or_unpack_device(N, K, bits, packed, codes2) == 0);
                CHECK(memcmp(codes, codes2, N * K) == 0);
                if (!zm) {
                    or_pack_zeros(N, K / g, bits, zeros, pz);
                    or_unpack_zeros(N, K / g, bits, pz, zeros2);
                    CHECK(memcmp(zeros, zeros2, N * (K / g)) == 0);
                    or_linear(M, N, K, g, x, K, codes, scales, zeros, rowptr, col, val, r, N);
                    or_linear(M, N, K, g, x, K, codes, scales, zeros, NULL, NULL, NULL, r, N);
                }
            }
    CHECK(or_pack_device(N, 300, 4, codes, packed) != 0); /* k % 256 != 0 is refused */

    /* expert FFN: 3 experts, D = F = 128, top-2 */
    enum { E = 3, D = 128, F = 128, T = 3 };
    uint8_t *ec = malloc(E * F * D), *ez = malloc(E * F);
    uint16_t *es = malloc(sizeof(uint16_t) * E * F);
    for (int i = 0; i < E * F * D; ++i) ec[i] = (uint8_t)(urand() * 16);
    for (int i = 0; i < E * F; ++i) {
        ez[i] = 8;
        es[i] = or_round_half(0.01);
    }
    int32_t ids[T * 2] = {0, 1, 2, 0, 1, 2};
    float wts[T * 2] = {0.5f, 0.25f, 0.5f, 0.25f, 0.75f, 0.1f};
    double *ro = malloc(sizeof(double) * T * D);
    or_moe_ffn(T, D, F, 2, 128, ids, wts, x, ec, es, ez, ec, es, ez, ec, es, ez, ro);

    /* quantized KV cache: layout round trips and decode attention with ragged, empty and
     * over-capacity lengths */
    enum { B = 2, HKV = 2, HQ = 4, CAP = 64 };
    const int64_t rows = (int64_t)B * HKV * CAP;
    uint16_t *kv = malloc(sizeof(uint16_t) * rows * 128);
    for (int64_t i = 0; i < rows * 128; ++i) kv[i] = hrand(1.5);
    int64_t *slot = malloc(sizeof(int64_t) * rows);
    for (int64_t i = 0; i < rows; ++i) slot[i] = i;
    uint8_t *kc = malloc(rows * 128), *vc = malloc(rows * 128), *back = malloc(rows * 128);
    float *ks = malloc(sizeof(float) * rows * 4), *vs = malloc(sizeof(float) * rows * 4);
    uint8_t *cache = calloc(rows * 128, 1);
    for (int bits = 4; bits <= 8; bits += 4)
        for (int which = 0; which <= 1; ++which) {
            or_kv_quantize_rows(kv, rows, 32, bits, kc, ks);
            or_kv_layout(which, bits, CAP, rows, slot, kc, cache);
            or_kv_unlayout(which, bits, CAP, rows, slot, cache, back);
            CHECK(memcmp(kc, back, rows * 128) == 0);
        }
    or_kv_quantize_rows(kv, rows, 32, 4, kc, ks);
    or_kv_quantize_rows(kv, rows, 64, 8, vc, vs);
    uint16_t qv[B * HQ * 128];
    for (int i = 0; i < B * HQ * 128; ++i) qv[i] = hrand(1.0);
    int32_t lens[B] = {CAP + 50, 0};
    double *o = malloc(sizeof(double) * B * HQ * 128), *a = malloc(sizeof(double) * B * HQ * 128);
    or_attn_decode(B, HQ, HKV, CAP, 4, 32, 8, 64, qv, kc, ks, vc, vs, lens, 0.088, o, a);
    lens[0] = 17;
    lens[1] = -3;
    or_attn_decode(B, HQ, HKV, CAP, 4, 32, 8, 64, qv, kc, ks, vc, vs, lens, 0.088, o, a);

    free(w); free(x); free(codes); free(codes2); free(packed); free(scales); free(zeros); free(zeros2); free(pz);
    free(r); free(ec); free(ez); free(es); free(ro); free(kv); free(slot); free(kc); free(vc); free(back);
    free(ks); free(vs); free(cache); free(o); free(a);
    printf("oracle driver ok\n");
    return 0;
}
