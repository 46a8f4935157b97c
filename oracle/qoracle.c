/*
 * qoracle.c -- plain, slow, obviously-correct CPU reference for the weight-only
 * mixed-bit quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this
 * file; only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * use it.  It shares no code, header or table with the GPU library.
 *
 * Sources (pages cited by title and section):
 *  [MB]  "二三五六" mixed 2/3/5/6-bit quantization with CPU/GPU hybrid inference
 *        (pwwt.cn): s2.3 block size and scale overhead; s3.1 packing units (smallest n
 *        with n*b divisible by 8); s3.2 unpack shift sequences, little-endian reads;
 *        s4.2 fp32 scale multiply.
 *  [IA]  inference acceleration guide (mzlw.cn): s1.1 the affine mapping
 *        scale=(max-min)/(qmax-qmin), zero_point=qmin-round(min/scale),
 *        q=round(x/scale)+zero_point, x_hat=(q-zero_point)*scale.
 *  [70B] single-GPU 70B five-layer stack (bjdmk.com.cn/5414039): s2 group-wise
 *        outlier-aware INT4 (groups of 128, top 0.1% |w| held out in fp16, added back
 *        after the GEMM); s3 unfused reference path dequantize -> matmul(x, W^T).
 *  [KV]  KV-cache INT8/INT4 quantization (kwkr.cn): s1.1, s3.1-s3.3 byte sums; s2.1
 *        symmetric absmax scale; s2.2 per-group along the head dimension; s2.3 K at
 *        INT4 with V at INT8; s3.1 FP32 scales; s5.1 4-bit packing, the operator
 *        consuming the quantized cache directly.
 *  [MoE] on-device MoE memory wall (bjdmk.com.cn/5648983): s1.1 weight/KV byte
 *        formulas; s4.2 routed expert tasks (hidden states + top-k expert ids).
 *  [IA]  also s1.2: W8A8 (weights and activations in INT8 on the integer matrix units, with
 *        dynamic per-token activation quantization); [MB] s4.2: unpack to 8-bit integers,
 *        integer dot-product accumulate, scale in floating point.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - codes are unsigned 0..2^b-1, round() is round-half-to-even, q and zp clamp to
 *    [0, qmax];
 *  - the group range [lo, hi] is extended to contain 0 so zp always fits b bits;
 *  - scale, zero point and codes are computed in IEEE fp32 (no fused multiply-add)
 *    from the fp16-rounded scale; an all-zero group gets scale 1.0, zp 0; a scale that
 *    rounds to zero or an fp16 subnormal is raised to 2^-14;
 *  - "top 0.1% per group" is read as the global floor(frac*N*K) largest |w| (fp16
 *    magnitude, ties to the lower row-major index), removed from the group range by
 *    setting them to +0 in the dense copy and kept in an fp16 CSR over W's rows;
 *  - bits inside a packing unit are LSB-first and units are stored little-endian;
 *  - symmetric groups ([MB] s2.3: no zero point stored at low bit widths, the scale
 *    absorbs the offset): the range is [-m, m] with m = max |w|, so the scale is
 *    fp16((m + m) / qmax) and the zero point is the midpoint 2^(b-1), which the
 *    asymmetric formula would also give for that range; it is implied, not stored, and
 *    an all-zero group gets scale 1.0 with every code at the midpoint;
 *  - zero points stored in b bits ([MB] s2.3): the same zero points as the affine groups,
 *    row n a little-endian stream of b-bit fields (LSB-first), rows padded to 32-bit words;
 *  - fp8 block scales with an fp16 fallback ([MB] s2.3): E4M3 (sign, 4-bit exponent with
 *    bias 7, 3-bit mantissa, no infinities, 0x7F NaN) times one fp32 factor per row,
 *    F = (largest fp32 group scale of the row) * 2^-8 (exact: the largest group maps to 256);
 *    a group's code is the smallest E4M3 value >= s32 / F, the stored scale F * value, and
 *    groups with s32 / F below E4M3's normal range (2^-6) keep the fp16 scale of the fp16
 *    path, marked by a code
 *    with the sign bit set whose low 7 bits index the row's fallback list; all-zero groups
 *    store code 0; codes and zero points are computed from the stored scale;
 *  - KV cache ([KV] s2.1-s2.2, s3.1): symmetric groups along the head dimension with
 *    qmax = 2^(b-1) - 1, an fp32 scale m / qmax, codes rint(x / s) clamped to
 *    [-qmax, qmax] and stored offset by 2^(b-1); an all-zero group stores scale 0;
 *    attention over an empty sequence returns 0.
 *
 * Arithmetic: quantization in fp32 exactly as stated; every matmul accumulates in
 * fp64 over the exactly dequantized weights.  Build: gcc -O2 -ffp-contract=off
 * -fno-fast-math -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary64                                                  */
/* ------------------------------------------------------------------------------ */

/* Value of a binary16 bit pattern: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double or_half_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* Table of or_half_value over all 65536 patterns (filled once from the definition above;
 * a speed convenience for the large sampled checks, same values). */
static double g_half_table[65536];
static int g_half_table_ready;

static double hv(uint16_t h)
{
    if (!g_half_table_ready) {
        for (int i = 0; i < 65536; ++i) g_half_table[i] = or_half_value((uint16_t)i);
        g_half_table_ready = 1;
    }
    return g_half_table[h];
}

/* Round a binary64 value to the nearest binary16, ties to even (one rounding). */
uint16_t or_round_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7E00;
    if (a >= 65520.0)                 /* at or above the midpoint 65504..65536 */
        return sign | 0x7C00;
    if (a < 0x1p-14) {                /* subnormal range: integer multiples of 2^-24 */
        double q = nearbyint(a * 0x1p24);
        return sign | (uint16_t)q;    /* q == 1024 is the smallest normal, correctly */
    }
    int e;
    double m = frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                    /* a = (2m) * 2^E, 2m in [1, 2) */
    double frac = nearbyint((2.0 * m - 1.0) * 1024.0);
    if (frac == 1024.0) {
        frac = 0.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | (int)frac);
}

/* ------------------------------------------------------------------------------ */
/* Group quantizer  ([IA] s1.1; [70B] s2 groups of 128; [MB] s2.3 fp16 scale)       */
/* ------------------------------------------------------------------------------ */

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Quantize one group of `n` fp16 weights (already with outliers set to +0). */
void or_quantize_group(const uint16_t *w, int n, int bits,
                       uint16_t *scale_out, uint8_t *zero_out, uint8_t *codes_out)
{
    const int qmin = 0, qmax = (1 << bits) - 1;
    float lo = 0.0f, hi = 0.0f;                      /* range always contains 0 */
    for (int i = 0; i < n; ++i) {
        float v = (float)hv(w[i]);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    if (hi == lo) {                                  /* all-zero group */
        *scale_out = 0x3C00;                         /* 1.0 */
        *zero_out = 0;
        for (int i = 0; i < n; ++i) codes_out[i] = 0;
        return;
    }
    volatile float range = hi - lo;                  /* fp32, rounded */
    volatile float s32 = range / (float)(qmax - qmin);
    uint16_t sh = or_round_half((double)s32);
    if ((sh & 0x7C00) == 0)                          /* zero or subnormal fp16 */
        sh = 0x0400;                                 /* 2^-14 */
    float sf = (float)or_half_value(sh);
    volatile float lo_over_s = lo / sf;
    int zp = clampi(qmin - (int)rintf(lo_over_s), qmin, qmax);
    for (int i = 0; i < n; ++i) {
        volatile float t = (float)hv(w[i]) / sf;
        codes_out[i] = (uint8_t)clampi((int)rintf(t) + zp, qmin, qmax);
    }
    *scale_out = sh;
    *zero_out = (uint8_t)zp;
}

/* Quantize one symmetric group of `n` fp16 weights: zero point 2^(bits-1), implied. */
void or_quantize_group_sym(const uint16_t *w, int n, int bits, uint16_t *scale_out, uint8_t *codes_out)
{
    const int qmax = (1 << bits) - 1, z = 1 << (bits - 1);
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf((float)hv(w[i]));
        if (a > m) m = a;
    }
    if (m == 0.0f) {                                 /* all-zero group */
        *scale_out = 0x3C00;                         /* 1.0 */
        for (int i = 0; i < n; ++i) codes_out[i] = (uint8_t)z;
        return;
    }
    volatile float two_m = m + m;                    /* exact */
    volatile float s32 = two_m / (float)qmax;
    uint16_t sh = or_round_half((double)s32);
    if ((sh & 0x7C00) == 0)                          /* zero or subnormal fp16 */
        sh = 0x0400;                                 /* 2^-14 */
    float sf = (float)or_half_value(sh);
    for (int i = 0; i < n; ++i) {
        volatile float t = (float)hv(w[i]) / sf;
        codes_out[i] = (uint8_t)clampi((int)rintf(t) + z, 0, qmax);
    }
    *scale_out = sh;
}

/* Number of outliers held out for a fraction `frac` of an N x K matrix. */
int64_t or_outlier_count(int64_t n, int64_t k, double frac)
{
    if (!(frac > 0.0)) return 0;
    return (int64_t)floor(frac * (double)(n * k));
}

/* qsort comparator state: rank by fp16 magnitude descending, then index ascending. */
static const uint16_t *g_rank_w;
static int64_t g_rank_k, g_rank_ldw;

static int rank_cmp(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    uint16_t ma = g_rank_w[(a / g_rank_k) * g_rank_ldw + a % g_rank_k] & 0x7FFF;
    uint16_t mb = g_rank_w[(b / g_rank_k) * g_rank_ldw + b % g_rank_k] & 0x7FFF;
    if (ma != mb) return ma > mb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/*
 * Quantize an N x K fp16 matrix (row n = output feature, groups of `g` consecutive k).
 * With outlier_frac > 0 the floor(frac*N*K) largest |w| are held out ([70B] s2):
 * their dense slots become +0 before the group range is taken, and the original fp16
 * values go to a CSR over rows (cols ascending).  Returns 0 on success, 1 if the CSR
 * capacity is too small (*nnz_out then holds the required count), 2 on bad arguments.
 * zero_mode 1 quantizes symmetric groups (zeros is then not written and may be NULL).
 */
int or_quantize(int64_t N, int64_t K, int bits, int g, int zero_mode,
                const uint16_t *w, int64_t ldw, double outlier_frac,
                uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                int32_t *rowptr, int32_t *col, uint16_t *val, int64_t cap, int64_t *nnz_out)
{
    if (bits < 2 || bits > 6 || g <= 0 || K % g != 0 || ldw < K || zero_mode < 0 || zero_mode > 1) return 2;
    int64_t kout = or_outlier_count(N, K, outlier_frac);
    *nnz_out = kout;
    if (kout > 0 && kout > cap) return 1;

    uint8_t *held = NULL;
    if (kout > 0) {
        int64_t total = N * K;
        int64_t *idx = (int64_t *)malloc((size_t)total * sizeof(int64_t));
        held = (uint8_t *)calloc((size_t)total, 1);
        for (int64_t i = 0; i < total; ++i) idx[i] = i;
        g_rank_w = w; g_rank_k = K; g_rank_ldw = ldw;
        qsort(idx, (size_t)total, sizeof(int64_t), rank_cmp);
        for (int64_t i = 0; i < kout; ++i) held[idx[i]] = 1;
        free(idx);
    }
    if (rowptr) {
        int64_t p = 0;
        rowptr[0] = 0;
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                if (held && held[n * K + k]) {
                    col[p] = (int32_t)k;
                    val[p] = w[n * ldw + k];
                    ++p;
                }
            }
            rowptr[n + 1] = (int32_t)p;
        }
    }
    int64_t G = K / g;
    uint16_t *buf = (uint16_t *)malloc((size_t)g * sizeof(uint16_t));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t gi = 0; gi < G; ++gi) {
            for (int i = 0; i < g; ++i) {
                int64_t k = gi * g + i;
                buf[i] = (held && held[n * K + k]) ? 0x0000 : w[n * ldw + k];
            }
            if (zero_mode == 1)
                or_quantize_group_sym(buf, g, bits, &scales[n * G + gi], &codes[n * K + gi * g]);
            else
                or_quantize_group(buf, g, bits, &scales[n * G + gi], &zeros[n * G + gi],
                                  &codes[n * K + gi * g]);
        }
    }
    free(buf);
    free(held);
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* fp8 block scales with an fp16 fallback  ([MB] s2.3)                              */
/* ------------------------------------------------------------------------------ */

/* Value of an E4M3 byte (OCP 8-bit float, "FN" variant): sign bit, exponent bits 6..3 with
 * bias 7, mantissa bits 2..0; exponent 0 is subnormal (mantissa/8 * 2^-6); 0x7F and 0xFF are
 * NaN; there are no infinities (0x7E = 448 is the largest finite value). */
double or_e4m3_value(int code)
{
    const int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return sign ? -mag : mag;
}

/* The smallest positive finite E4M3 code whose value is >= t (t > 0), or -1 if t > 448:
 * a scan of the codes in increasing value. */
int or_e4m3_ceil(float t)
{
    for (int c = 0x01; c <= 0x7E; ++c)
        if (or_e4m3_value(c) >= (double)t) return c;
    return -1;
}

/* One row of K weights in groups of g with fp8 scales.  Writes the codes (u8 [K]), the scale
 * bytes (u8 [K/g]), the zero points (u8 [K/g]; midpoints for sym), the stored scale of each
 * group as fp32 (scale_out [K/g]: F * E4M3 value, the fp16 fallback's value, or 0 for an
 * all-zero group), the row factor F and up to fb_cap fallback fp16 scales; returns the
 * number of fallback groups of the row. */
int or_quantize_fp8_row(int64_t K, int bits, int g, int sym, const uint16_t *w, uint8_t *codes, uint8_t *sc8,
                        uint8_t *zeros, float *scale_out, float *factor, uint16_t *fb, int fb_cap)
{
    const int qmax = (1 << bits) - 1, mid = 1 << (bits - 1);
    const int64_t G = K / g;
    float *s32 = (float *)malloc(sizeof(float) * (size_t)G);
    float *lo = (float *)malloc(sizeof(float) * (size_t)G);
    int *zero = (int *)malloc(sizeof(int) * (size_t)G);
    float mx = 0.0f;
    int any = 0;
    /* the fp32 scale of every group, as in the fp16 path before its fp16 rounding */
    for (int64_t gi = 0; gi < G; ++gi) {
        const uint16_t *wg = w + gi * g;
        float l = 0.0f, h = 0.0f, m = 0.0f;
        for (int i = 0; i < g; ++i) {
            const float v = (float)hv(wg[i]);
            if (v < l) l = v;
            if (v > h) h = v;
            if (fabsf(v) > m) m = fabsf(v);
        }
        lo[gi] = l;
        zero[gi] = sym ? (m == 0.0f) : (h == l);
        if (zero[gi]) continue;
        volatile float range = sym ? m + m : h - l;
        volatile float s = range / (float)qmax;
        s32[gi] = s;
        if (!any || s > mx) mx = s;
        any = 1;
    }
    volatile float F = any ? mx * 0.00390625f : 1.0f;  /* exact: times 2^-8 */
    *factor = F;
    int nfb = 0;
    for (int64_t gi = 0; gi < G; ++gi) {
        const uint16_t *wg = w + gi * g;
        uint8_t *cg = codes + gi * g;
        if (zero[gi]) {
            sc8[gi] = 0;
            scale_out[gi] = 0.0f;
            zeros[gi] = (uint8_t)(sym ? mid : 0);
            for (int i = 0; i < g; ++i) cg[i] = (uint8_t)(sym ? mid : 0);
            continue;
        }
        volatile float t = s32[gi] / F;
        const int c = (t >= 0.015625f) ? or_e4m3_ceil(t) : -1;
        float sf;
        if (c > 0) {
            volatile float prod = F * (float)or_e4m3_value(c);
            sf = prod;
            sc8[gi] = (uint8_t)c;
        } else {  /* below E4M3's normal range: the fp16 path's scale */
            uint16_t sh = or_round_half((double)s32[gi]);
            if ((sh & 0x7C00) == 0) sh = 0x0400;
            sf = (float)or_half_value(sh);
            if (nfb < fb_cap) fb[nfb] = sh;
            sc8[gi] = (uint8_t)(0x80 | (nfb & 0x7F));
            ++nfb;
        }
        scale_out[gi] = sf;
        int zp = mid;
        if (!sym) {
            volatile float lo_over_s = lo[gi] / sf;
            zp = clampi(-(int)rintf(lo_over_s), 0, qmax);
        }
        zeros[gi] = (uint8_t)zp;
        for (int i = 0; i < g; ++i) {
            volatile float q = (float)hv(wg[i]) / sf;
            cg[i] = (uint8_t)clampi((int)rintf(q) + zp, 0, qmax);
        }
    }
    free(s32);
    free(lo);
    free(zero);
    return nfb;
}

/* Every row of W [N][K] (stride ldw); fb is [N][fb_stride]; counts [N] receives each row's
 * number of fallback groups.  Returns the largest count. */
int or_quantize_fp8(int64_t N, int64_t K, int bits, int g, int sym, const uint16_t *w, int64_t ldw, uint8_t *codes,
                    uint8_t *sc8, uint8_t *zeros, float *scales, float *factors, uint16_t *fb, int fb_stride,
                    int32_t *counts)
{
    const int64_t G = K / g;
    int most = 0;
    for (int64_t n = 0; n < N; ++n) {
        counts[n] = or_quantize_fp8_row(K, bits, g, sym, w + n * ldw, codes + n * K, sc8 + n * G, zeros + n * G,
                                        scales + n * G, factors + n, fb + n * fb_stride, fb_stride);
        if (counts[n] > most) most = counts[n];
    }
    return most;
}

/* ------------------------------------------------------------------------------ */
/* Packing units  ([MB] s3.1, s3.2)                                                */
/* ------------------------------------------------------------------------------ */

/* Values per unit: smallest n with n*b divisible by 8. */
int or_unit_values(int bits)
{
    int n = 1;
    while ((n * bits) % 8 != 0) ++n;
    return n;
}

int or_unit_bytes(int bits) { return or_unit_values(bits) * bits / 8; }

/* One unit: value i sits at bits [b*i, b*i+b) of the little-endian integer formed by
 * the unit's bytes (the shift sequences 0,3,...,21 / 0,6,12,18 / 5i of [MB] s3.2). */
static void pack_unit(const uint8_t *codes, int bits, uint8_t *out)
{
    int nv = or_unit_values(bits), nb = or_unit_bytes(bits);
    uint64_t v = 0;
    for (int i = 0; i < nv; ++i) v |= (uint64_t)codes[i] << (bits * i);
    for (int j = 0; j < nb; ++j) out[j] = (uint8_t)(v >> (8 * j));
}

static void unpack_unit(const uint8_t *in, int bits, uint8_t *codes)
{
    int nv = or_unit_values(bits), nb = or_unit_bytes(bits);
    uint64_t v = 0;
    for (int j = 0; j < nb; ++j) v |= (uint64_t)in[j] << (8 * j);
    uint64_t mask = ((uint64_t)1 << bits) - 1;
    for (int i = 0; i < nv; ++i) codes[i] = (uint8_t)((v >> (bits * i)) & mask);
}

/* Canonical layout: each row n is K*b/8 bytes of consecutive units in k order. */
void or_pack_canonical(int64_t N, int64_t K, int bits, const uint8_t *codes, uint8_t *out)
{
    int nv = or_unit_values(bits), nb = or_unit_bytes(bits);
    int64_t rowbytes = K * bits / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t u = 0; u < K / nv; ++u)
            pack_unit(&codes[n * K + u * nv], bits, &out[n * rowbytes + u * nb]);
}

void or_unpack_canonical(int64_t N, int64_t K, int bits, const uint8_t *in, uint8_t *codes)
{
    int nv = or_unit_values(bits), nb = or_unit_bytes(bits);
    int64_t rowbytes = K * bits / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t u = 0; u < K / nv; ++u)
            unpack_unit(&in[n * rowbytes + u * nb], bits, &codes[n * K + u * nv]);
}

/*
 * Device layout: the library's own tile order, defined here from its documented statement.
 * Three steps, each invertible:
 *  1. value order inside packing groups.  The GPU turns two codes into one fp16 pair with a
 *     single mask when the two sit 16 bits apart, so inside each group of G values (pair
 *     p = values 2p and 2p+1) packed position p < G/2 holds value 2p and position G/2 + p
 *     holds value 2p + 1.  Groups: 4 consecutive k for 6 bits (one 3-byte unit); 8
 *     consecutive k for 3, 4 and 5 bits (one 8-k block); for 2 bits the two 8-k blocks that
 *     start at k0 and k0 + 32 with k0 % 64 < 32 (16 values, k0.. then k0+32..);
 *  2. canonical unit packing (LSB first, little endian) of the reordered codes;
 *  3. a byte map of the canonical bytes (units stay whole):
 *     - 16-row x 256-k tiles, row-block major then k-tile; tile size 512*b bytes;
 *     - inside a tile, "lane" l = 16*t + r (r = row in block, t = 0..3) owns a chunk of
 *       8 blocks of 8 consecutive k (b bytes each, canonical bytes in order); block j
 *       (0..7) covers k0 = 256*kt + 128*(j/4) + 32*(j%4) + 8*t;
 *     - chunk byte c sits at 1024*(c/16) + 16*l + c%16 while c < F = 16*floor(b/2),
 *       and at 64*F + 8*l + (c-F) for the 8-byte tail of odd b.
 */
static int dev_group_size(int bits) { return bits == 2 ? 16 : bits == 6 ? 4 : 8; }

/* k of value i of the group that starts at k0 (k0 is the group's first k). */
static int64_t dev_group_k(int bits, int64_t k0, int i)
{
    if (bits == 2) return i < 8 ? k0 + i : k0 + 32 + (i - 8);
    return k0 + i;
}

/* Is k0 the first k of a group? */
static int dev_group_start(int bits, int64_t k0)
{
    if (bits == 2) return k0 % 8 == 0 && k0 % 64 < 32;
    return k0 % dev_group_size(bits) == 0;
}

/* Value (index inside its group) held at packed position p. */
static int dev_group_value(int G, int p) { return p < G / 2 ? 2 * p : 2 * (p - G / 2) + 1; }

/* Step 1 on a whole row-major [N][K] code array (inverse if `inverse`). */
static void dev_reorder(int64_t N, int64_t K, int bits, const uint8_t *in, uint8_t *out, int inverse)
{
    int G = dev_group_size(bits);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k0 = 0; k0 < K; ++k0) {
            if (!dev_group_start(bits, k0)) continue;
            for (int p = 0; p < G; ++p) {
                int64_t kp = dev_group_k(bits, k0, p), kv = dev_group_k(bits, k0, dev_group_value(G, p));
                if (!inverse)
                    out[n * K + kp] = in[n * K + kv];   /* position p <- value */
                else
                    out[n * K + kv] = in[n * K + kp];
            }
        }
}

/* Step 3: byte offset of canonical byte `cb` of row `n`. */
int64_t or_device_offset(int64_t n, int64_t cb, int64_t K, int bits)
{
    int64_t k0 = (cb / bits) * 8;          /* first k of the 8-k block holding cb */
    int64_t bib = cb % bits;               /* byte inside the block */
    int64_t rb = n / 16, r = n % 16;
    int64_t kt = k0 / 256, kk = k0 % 256;
    int64_t gi = kk / 128, kq = kk % 128;
    int64_t j4 = kq / 32, t = (kq % 32) / 8;
    int64_t lane = 16 * t + r;
    int64_t j = 4 * gi + j4;
    int64_t c = bits * j + bib;
    int64_t F = 16 * (bits / 2);
    int64_t tile = rb * (K / 256) + kt;
    int64_t off = c < F ? 1024 * (c / 16) + 16 * lane + c % 16 : 64 * F + 8 * lane + (c - F);
    return tile * 512 * bits + off;
}

/* Steps 1 and 2 only: the canonical bytes that step 3 moves. */
void or_device_reorder(int64_t N, int64_t K, int bits, const uint8_t *codes, uint8_t *out, int inverse)
{
    dev_reorder(N, K, bits, codes, out, inverse);
}

int or_pack_device(int64_t N, int64_t K, int bits, const uint8_t *codes, uint8_t *out)
{
    if (N % 16 != 0 || K % 256 != 0) return 2;
    int64_t rowbytes = K * bits / 8;
    uint8_t *perm = (uint8_t *)malloc((size_t)(N * K));
    uint8_t *canon = (uint8_t *)malloc((size_t)(N * rowbytes));
    dev_reorder(N, K, bits, codes, perm, 0);
    or_pack_canonical(N, K, bits, perm, canon);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t cb = 0; cb < rowbytes; ++cb)
            out[or_device_offset(n, cb, K, bits)] = canon[n * rowbytes + cb];
    free(canon);
    free(perm);
    return 0;
}

int or_unpack_device(int64_t N, int64_t K, int bits, const uint8_t *in, uint8_t *codes)
{
    if (N % 16 != 0 || K % 256 != 0) return 2;
    int64_t rowbytes = K * bits / 8;
    uint8_t *canon = (uint8_t *)malloc((size_t)(N * rowbytes));
    uint8_t *perm = (uint8_t *)malloc((size_t)(N * K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t cb = 0; cb < rowbytes; ++cb)
            canon[n * rowbytes + cb] = in[or_device_offset(n, cb, K, bits)];
    or_unpack_canonical(N, K, bits, canon, perm);
    dev_reorder(N, K, bits, perm, codes, 1);
    free(perm);
    free(canon);
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* Linear layer  ([70B] s3 unfused path; [IA] s1.1 dequantize; [70B] s2 add-back)   */
/* ------------------------------------------------------------------------------ */

/* Exact dequantized weight (q - zp) * s, in fp64. */
static double dequant(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                      int64_t K, int g, int64_t n, int64_t k)
{
    int64_t G = K / g;
    return ((double)codes[n * K + k] - (double)zeros[n * G + k / g]) *
           hv(scales[n * G + k / g]);
}

/*
 * r[m, n] = sum_k x[m, k] * What[n, k] + sum_{(n, k) in CSR} x[m, k] * val,
 * y = x * What^T with What = dequantize(codes, scales, zeros), accumulated in fp64.
 * CSR pointers may be NULL (no outliers).
 */
void or_linear(int64_t M, int64_t N, int64_t K, int g,
               const uint16_t *x, int64_t ldx,
               const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
               const int32_t *rowptr, const int32_t *col, const uint16_t *val,
               double *r, int64_t ldr)
{
    (void)hv(0);  /* fill the table before the parallel loop */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += hv(x[m * ldx + k]) * dequant(codes, scales, zeros, K, g, n, k);
            if (rowptr)
                for (int32_t p = rowptr[n]; p < rowptr[n + 1]; ++p)
                    acc += hv(x[m * ldx + col[p]]) * hv(val[p]);
            r[m * ldr + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------------ */
/* Routed experts  ([MoE] s4.2: hidden states + top-k expert ids per token)         */
/* ------------------------------------------------------------------------------ */

static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * SwiGLU intermediate of one token through one expert, before its fp16 rounding:
 * v[f] = silu(g_f) * u_f, g = What_gate x, u = What_up x, all in fp64 ([MoE] s4.2 expert
 * FFN gate/up; silu(v) = v / (1 + e^-v)).  Gate/up codes [F][D], scales/zeros [F][D/g].
 */
void or_swiglu_act(int64_t D, int64_t F, int g, const uint16_t *xt,
                   const uint8_t *gc, const uint16_t *gs, const uint8_t *gz,
                   const uint8_t *uc, const uint16_t *us, const uint8_t *uz, double *v)
{
    (void)hv(0);
#pragma omp parallel for schedule(static)
    for (int64_t f = 0; f < F; ++f) {
        double gv = 0.0, uv = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double xv = hv(xt[d]);
            gv += xv * dequant(gc, gs, gz, D, g, f, d);
            uv += xv * dequant(uc, us, uz, D, g, f, d);
        }
        v[f] = silu(gv) * uv;
    }
}

/*
 * Per token t: out[t] = sum_j p[t][j] * FFN_{e}(x[t]), e = ids[t][j], with
 * FFN_e(x) = What_down_e * fp16( silu(What_gate_e x) * (What_up_e x) ).
 * Gate/up: codes [E][F][D], scales/zeros [E][F][D/g]; down: codes [E][D][F],
 * scales/zeros [E][D][F/g].  Accumulation in fp64; the SwiGLU product is rounded to
 * fp16 once (the down projection's input is an fp16 activation).  r is [T][D] fp64.
 */
void or_moe_ffn(int64_t T, int64_t D, int64_t F, int topk, int g,
                const int32_t *ids, const float *wts, const uint16_t *x,
                const uint8_t *gc, const uint16_t *gs, const uint8_t *gz,
                const uint8_t *uc, const uint16_t *us, const uint8_t *uz,
                const uint8_t *dc, const uint16_t *ds, const uint8_t *dz,
                double *r)
{
    (void)hv(0);
    double *v = (double *)malloc((size_t)F * sizeof(double));
    double *a = (double *)malloc((size_t)F * sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t d = 0; d < D; ++d) r[t * D + d] = 0.0;
        for (int j = 0; j < topk; ++j) {
            int64_t e = ids[t * topk + j];
            double p = (double)wts[t * topk + j];
            const int64_t gF = F * (D / g), gD = D * (F / g);
            or_swiglu_act(D, F, g, x + t * D, gc + e * F * D, gs + e * gF, gz + e * gF,
                          uc + e * F * D, us + e * gF, uz + e * gF, v);
            for (int64_t f = 0; f < F; ++f) a[f] = hv(or_round_half(v[f]));
            const uint8_t *dce = dc + e * D * F, *dze = dz + e * gD;
            const uint16_t *dse = ds + e * gD;
#pragma omp parallel for schedule(static)
            for (int64_t d = 0; d < D; ++d) {
                double o = 0.0;
                for (int64_t f = 0; f < F; ++f) o += a[f] * dequant(dce, dse, dze, F, g, d, f);
                r[t * D + d] += p * o;
            }
        }
    }
    free(v);
    free(a);
}

/* ------------------------------------------------------------------------------ */
/* Zero points stored in b bits  ([MB] s2.3)                                        */
/* ------------------------------------------------------------------------------ */

/* Bytes of one row of b-bit zero points: G fields, rounded up to whole 32-bit words. */
int64_t or_zero_row_bytes(int64_t G, int bits) { return 4 * ((G * bits + 31) / 32); }

/* [MB] s2.3 counts an asymmetric group's zero point at b bits.  Row n of the packed array
 * is a little-endian bit stream: zero point gi of the row occupies bits [gi*b, gi*b + b)
 * (LSB-first, as the page's units store codes), the rest of the row's last word is zero. */
void or_pack_zeros(int64_t N, int64_t G, int bits, const uint8_t *zeros, uint8_t *out)
{
    const int64_t rb = or_zero_row_bytes(G, bits);
    memset(out, 0, (size_t)(N * rb));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t gi = 0; gi < G; ++gi)
            for (int i = 0; i < bits; ++i) {
                const int64_t bit = gi * bits + i;
                if ((zeros[n * G + gi] >> i) & 1) out[n * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
}

void or_unpack_zeros(int64_t N, int64_t G, int bits, const uint8_t *in, uint8_t *zeros)
{
    const int64_t rb = or_zero_row_bytes(G, bits);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t gi = 0; gi < G; ++gi) {
            unsigned v = 0;
            for (int i = 0; i < bits; ++i) {
                const int64_t bit = gi * bits + i;
                v |= (unsigned)((in[n * rb + bit / 8] >> (bit % 8)) & 1) << i;
            }
            zeros[n * G + gi] = (uint8_t)v;
        }
}

/* ------------------------------------------------------------------------------ */
/* Quantized KV cache and decode attention  ([KV] s2.1-s2.3, s3.1, s5.1)             */
/* ------------------------------------------------------------------------------ */

/* Symmetric per-group quantization of one cached row ([KV] s2.1: the scale comes from
 * the absolute maximum, every element is divided by it and rounded; s2.2: adjacent
 * elements of the head dimension share one scale per group; s3.1: the scale is FP32).
 * Readings: qmax = 2^(b-1) - 1 (127 at 8 bits, the [-127, 127] range of the inference
 * guide's INT8 example; 7 at 4 bits); s = m / qmax in IEEE fp32; q = rint(x / s) with
 * ties to even, clamped to [-qmax, qmax]; an all-zero group stores s = 0 and q = 0.
 * Codes are stored offset by 2^(b-1) (so 1 .. 2^b - 1; 2^(b-1) means 0). */
void or_kv_quantize_row(const uint16_t *x, int n, int g, int bits, uint8_t *codes, float *scales)
{
    const int qmax = (1 << (bits - 1)) - 1, mid = 1 << (bits - 1);
    for (int g0 = 0; g0 < n; g0 += g) {
        float m = 0.0f;
        for (int i = 0; i < g; ++i) {
            const float a = fabsf((float)hv(x[g0 + i]));
            if (a > m) m = a;
        }
        const float s = m / (float)qmax;
        scales[g0 / g] = m == 0.0f ? 0.0f : s;
        for (int i = 0; i < g; ++i) {
            int q = 0;
            if (m != 0.0f) {
                const float v = (float)hv(x[g0 + i]) / s;
                q = clampi((int)rintf(v), -qmax, qmax);
            }
            codes[g0 + i] = (uint8_t)(q + mid);
        }
    }
}

/* or_kv_quantize_row over `rows` consecutive rows of 128 values. */
void or_kv_quantize_rows(const uint16_t *x, int64_t rows, int g, int bits, uint8_t *codes, float *scales)
{
    for (int64_t i = 0; i < rows; ++i)
        or_kv_quantize_row(x + i * 128, 128, g, bits, codes + i * 128, scales + i * (128 / g));
}

/* Storage of the quantized cache (the library's own encoding; the page fixes only that
 * 4-bit values pack two per byte, [KV] s5.1).  Positions are in values: value p of a
 * 4-bit stream is the low nibble of byte p/2 when p is even, the high nibble otherwise.
 *  sigma(s): slot s = 0..7 of an 8-value piece sits at s (8-bit) or s/2 + 4*(s%2)
 *  (4-bit: the two values of a pair are four nibbles apart).
 *  K row (one token, head_dim 128): value d = 32j + 8t + s sits at 32t + 8j + sigma(s).
 *  V tile (32 tokens x 128, tile u holds tokens 32u .. 32u+31 of one head): token
 *  tau = 32u + w and value d = 16c + r, with w = 4t + s (s < 4) or 16 + 4t + (s - 4)
 *  (s >= 4), belong to lane l = 16t + r, slice c, slot s.  A lane's eight 8-value slices
 *  fill its pieces of P = 128/b values (P/8 slices each), and piece e of lane l sits at
 *  64*P*e + P*l: value position 64*P*(c / (P/8)) + P*l + 8*(c % (P/8)) + sigma(s). */
static int kv_sigma(int bits, int s) { return bits == 8 ? s : s / 2 + 4 * (s % 2); }

int64_t or_kv_k_pos(int bits, int d)
{
    const int j = d / 32, t = (d % 32) / 8, s = d % 8;
    return 32 * t + 8 * j + kv_sigma(bits, s);
}

int64_t or_kv_v_pos(int bits, int w, int d)
{
    const int hi = w >= 16, t = ((w % 16) / 4), s = (w % 4) + 4 * hi;
    const int c = d / 16, r = d % 16, l = 16 * t + r;
    const int P = 128 / bits, spp = P / 8;
    return 64 * P * (c / spp) + P * l + 8 * (c % spp) + kv_sigma(bits, s);
}

static void put_value(uint8_t *base, int bits, int64_t pos, uint8_t v)
{
    if (bits == 8) {
        base[pos] = v;
    } else {
        uint8_t *b = base + pos / 2;
        *b = (pos % 2) ? (uint8_t)((*b & 0x0F) | (v << 4)) : (uint8_t)((*b & 0xF0) | (v & 0x0F));
    }
}

static uint8_t get_value(const uint8_t *base, int bits, int64_t pos)
{
    if (bits == 8) return base[pos];
    return (pos % 2) ? (uint8_t)(base[pos / 2] >> 4) : (uint8_t)(base[pos / 2] & 0x0F);
}

/* Value position of (row R = (b*heads + h)*cap + tau, d) in the cache of one tensor,
 * counted from the cache base (which: 0 = K rows, 1 = V tiles; cap % 32 == 0). */
static int64_t kv_pos(int which, int bits, int64_t cap, int64_t R, int d)
{
    if (which == 0) return R * 128 + or_kv_k_pos(bits, d);
    const int64_t region = R / cap, tau = R % cap;
    return region * cap * 128 + (tau / 32) * 32 * 128 + or_kv_v_pos(bits, (int)(tau % 32), d);
}

/* Scatter offset codes [rows][128] into the cache bytes at rows slot[i] (K or V layout). */
void or_kv_layout(int which, int bits, int64_t cap, int64_t rows, const int64_t *slot,
                  const uint8_t *codes, uint8_t *cache)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int d = 0; d < 128; ++d)
            put_value(cache, bits, kv_pos(which, bits, cap, slot[i], d), codes[i * 128 + d]);
}

/* Gather: the inverse of or_kv_layout for rows slot[i]. */
void or_kv_unlayout(int which, int bits, int64_t cap, int64_t rows, const int64_t *slot,
                    const uint8_t *cache, uint8_t *codes)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int d = 0; d < 128; ++d)
            codes[i * 128 + d] = get_value(cache, bits, kv_pos(which, bits, cap, slot[i], d));
}

/* Decode attention over the quantized cache ([KV] s5.1: the operator reads the quantized
 * K/V and their scales directly).  For batch b and query head h (kv head h / (Hq/Hkv)),
 * over the first len[b] tokens of that kv head:
 *   z_t = sm_scale * sum_d q[h][d] * kq_t[d]*ks_t[d/kg],  p = softmax(z),
 *   o[h][d] = sum_t p_t * vq_t[d]*vs_t[d/vg]                      (all in fp64),
 * with kq, vq the signed codes (stored code - 2^(b-1)).  Also a[h][d] = sum_t p_t |v_t[d]|,
 * the weighted magnitude that bounds rounding errors of a computed o.  len[b] <= 0
 * gives o = 0, a = 0; a length above cap counts as cap (a sequence holds cap slots).
 * kc/vc: offset codes [B*Hkv*cap][128] (unpacked), ks/vs: [B*Hkv*cap][128/g] fp32;
 * q fp16 [B][Hq][128]. */
void or_attn_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t cap, int kbits, int kg, int vbits,
                    int vg, const uint16_t *q, const uint8_t *kc, const float *ks,
                    const uint8_t *vc, const float *vs, const int32_t *len, double sm_scale,
                    double *o, double *a)
{
    const int kmid = 1 << (kbits - 1), vmid = 1 << (vbits - 1);
    const int64_t grp = Hq / Hkv;
    (void)hv(0); /* fill the half table before the threads read it */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t hk = h / grp, base = (b * Hkv + hk) * cap;
            const int64_t L = len[b] > cap ? cap : len[b];
            double *oh = o + (b * Hq + h) * 128, *ah = a + (b * Hq + h) * 128;
            for (int d = 0; d < 128; ++d) oh[d] = ah[d] = 0.0;
            if (L <= 0) continue;
            double *z = (double *)malloc((size_t)L * sizeof(double));
            double zmax = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t R = base + t;
                double acc = 0.0;
                for (int d = 0; d < 128; ++d)
                    acc += hv(q[(b * Hq + h) * 128 + d]) *
                           ((double)((int)kc[R * 128 + d] - kmid) * (double)ks[R * (128 / kg) + d / kg]);
                z[t] = sm_scale * acc;
                if (z[t] > zmax) zmax = z[t];
            }
            double sum = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                z[t] = exp(z[t] - zmax);
                sum += z[t];
            }
            for (int64_t t = 0; t < L; ++t) {
                const int64_t R = base + t;
                const double p = z[t] / sum;
                for (int d = 0; d < 128; ++d) {
                    const double v = (double)((int)vc[R * 128 + d] - vmid) * (double)vs[R * (128 / vg) + d / vg];
                    oh[d] += p * v;
                    ah[d] += p * fabs(v);
                }
            }
            free(z);
        }
}

/* ------------------------------------------------------------------------------ */
/* Integer-dot path: int8 activations x b-bit weights  ([IA] s1.2; [MB] s4.2)       */
/* ------------------------------------------------------------------------------ */

/* Dynamic per-token activation quantization ([IA] s1.2: W8A8 quantizes activations to INT8
 * dynamically, per token).  Reading, as the symmetric INT8 form of [IA] s1.1 ([-127, 127]):
 * for row m, a = max_k |x[m][k]| in fp32, s = a / 127 in IEEE fp32, xq = clamp(rint(x / s),
 * -127, 127) (fp32 division, ties to even); an all-zero row stores s = 0 and xq = 0.
 * xq is row-major [M][K] here (the library's own k order inside each group is a storage
 * map, or_act_layout). */
void or_act_quantize(int64_t M, int64_t K, const uint16_t *x, int64_t ldx, int8_t *xq, float *scales)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * ldx;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf((float)hv(row[k]));
            if (v > a) a = v;
        }
        volatile float s = a / 127.0f;
        scales[m] = a == 0.0f ? 0.0f : s;
        for (int64_t k = 0; k < K; ++k) {
            int q = 0;
            if (a != 0.0f) {
                volatile float t = (float)hv(row[k]) / s;
                q = clampi((int)rintf(t), -127, 127);
            }
            xq[m * K + k] = (int8_t)q;
        }
    }
}

/* Position of k inside its 128-k group in the library's int8 activation rows: 16-byte pieces
 * (64-k step s, lane quarter t) holding k = 64s + 8t + [0, 8) then 64s + 32 + 8t + [0, 8), so
 * one 16-byte read gives a lane the 16 k values it multiplies on the integer matrix core. */
int64_t or_act_pos(int64_t k)
{
    const int64_t g = k / 128, kk = k % 128, st = kk / 64, rem = kk % 64;
    const int64_t p = rem / 32, t = (rem % 32) / 8, e = rem % 8;
    return g * 128 + 16 * (4 * st + t) + 8 * p + e;
}

/* Row-major xq [M][K] -> the library's storage order (inverse = 1: back). */
void or_act_layout(int64_t M, int64_t K, const int8_t *in, int8_t *out, int inverse)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            if (inverse) out[m * K + k] = in[m * K + or_act_pos(k)];
            else out[m * K + or_act_pos(k)] = in[m * K + k];
        }
}

/* r[m][n] = s_x[m] * sum_g s_w[n][g] * sum_{k in g} xq[m][k] * (q[n][k] - zp[n][g]) ([MB] s4.2:
 * integer dot products per group, the scale multiply in floating point), in fp64; every
 * group's integer sum is exact. */
void or_linear_a8(int64_t M, int64_t N, int64_t K, int g, const int8_t *xq, const float *sx,
                  const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, double *r)
{
    const int64_t G = K / g;
    (void)hv(0);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t gi = 0; gi < G; ++gi) {
                int64_t isum = 0;
                const int zp = zeros[n * G + gi];
                for (int64_t k = gi * g; k < (gi + 1) * g; ++k)
                    isum += (int64_t)xq[m * K + k] * ((int64_t)codes[n * K + k] - zp);
                acc += hv(scales[n * G + gi]) * (double)isum;
            }
            r[m * N + n] = (double)sx[m] * acc;
        }
}

/* ------------------------------------------------------------------------------ */
/* Byte accounting  ([MB] s1.2, s2.3; [KV] s1.1, s3.1-s3.3; [MoE] s1.1)             */
/* ------------------------------------------------------------------------------ */

/* Bytes of `numel` weights at `bits` with one scale (scale_bytes) and a zp of
 * zp_bits per group of g: numel*b/8 + (numel/g)*(scale_bytes + zp_bits/8). */
double or_quant_bytes(double numel, double bits, double g, double scale_bytes, double zp_bits)
{
    return numel * bits / 8.0 + (numel / g) * (scale_bytes + zp_bits / 8.0);
}

/* KV cache bytes: 2 (K and V) * layers * kv_heads * head_dim * tokens * bytes/elem. */
double or_kv_bytes(double layers, double kv_heads, double head_dim, double tokens,
                   double bytes_per_elem)
{
    return 2.0 * layers * kv_heads * head_dim * tokens * bytes_per_elem;
}

/* Threads the parallel loops above use from now on (n >= 1). */
void or_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads the parallel loops above use. */
int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
