// Host-side fused unpack + multiply-accumulate GEMV (the CPU half of a CPU/GPU layer split,
// 2/3/5/6-bit mixed quantization page, s4.1 and s4.3).  Host memory only.
//
// What the page asks of the CPU kernel, and how it is met here:
//  * unpacking fused into the multiply-accumulate loop, no intermediate buffer of unpacked
//    weights, the loop ordered by output so unpacked values are used at once (s4.1): each
//    thread takes R output rows at a time and walks k once, its unpacked codes living only in
//    vector registers;
//  * byte-permute unpacking on 256-bit vectors (s4.1): the 8 codes of an 8-k block (b bytes,
//    canonical page units) come from one 16-byte broadcast load, one byte shuffle that puts
//    the 4 bytes holding code i into 32-bit lane i, one per-lane variable shift and one mask --
//    the same four instructions for every width, straddling 3- and 5-bit fields included;
//    on CPUs with AVX-512 VBMI the same idea on 512-bit vectors: a byte permute, a variable
//    left shift and one ternary-logic op decode 16 codes straight to the fp32 values 1 + q/2^b;
//  * fp32 accumulation with the scale applied in fp32 (s4.2);
//  * software prefetch four cache lines ahead on every row stream (s4.3: distance 4);
//  * worker threads one fewer than the cores by default, leaving one for the scheduling side
//    (s5.2).
// The zero point is not subtracted per weight: per group, sum_k x_k (q_k - zp) = sum_k x_k q_k
// - zp * sum_k x_k, and the lane-wise sums of x are accumulated beside the products, so the
// inner loop is shuffle, shift, and, convert, and one fma per activation row.
#include <immintrin.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#include "qpack.h"

namespace qp {
qp_status fail(qp_status st, const char *fmt, ...);
}

namespace {

// IEEE binary16 -> binary32 (exact), for the portable path and the outlier values.
float half_to_float(uint16_t h)
{
    const uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31, f = h & 1023;
    uint32_t bits;
    if (e == 0) {
        if (f == 0) {
            bits = s;
        } else {  // subnormal: renormalise
            int sh = 0;
            uint32_t m = f;
            while (!(m & 1024)) {
                m <<= 1;
                ++sh;
            }
            bits = s | ((uint32_t)(113 - sh) << 23) | ((m & 1023) << 13);
        }
    } else if (e == 31) {
        bits = s | 0x7F800000u | (f << 13);
    } else {
        bits = s | ((e + 112) << 23) | (f << 13);
    }
    float v;
    memcpy(&v, &bits, 4);
    return v;
}

// binary32 -> binary16, round to nearest even (one rounding).
uint16_t float_to_half(float v)
{
    uint32_t x;
    memcpy(&x, &v, 4);
    const uint32_t s = (x >> 16) & 0x8000u;
    const int32_t e = (int32_t)((x >> 23) & 255) - 127;
    uint32_t m = x & 0x7FFFFFu;
    if (e == 128) return (uint16_t)(s | 0x7C00u | (m ? 0x200u : 0u));
    if (e > 15) return (uint16_t)(s | 0x7C00u);
    if (e >= -14) {  // normal range: keep 10 bits, round on the 13 dropped
        uint32_t h = ((uint32_t)(e + 15) << 10) | (m >> 13);
        const uint32_t rem = m & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  // may carry into the exponent
        return (uint16_t)(s | h);
    }
    if (e < -25) return (uint16_t)s;
    // subnormal result: value = (m | 2^23) * 2^(e-23), in units of 2^-24
    m |= 0x800000u;
    const int sh = -e - 1;  // 14..24
    uint32_t h = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(s | h);
}

struct HostArgs {
    const uint8_t *w;        // canonical packed rows, k*b/8 bytes each
    const uint16_t *scales;  // [n][G] fp16 scales, or null with fp8 scales:
    const uint8_t *sc8;      //   [n][G] scale bytes (E4M3 value, or 0x80 | fallback index)
    const float *rowf;       //   [n] row factors
    const uint16_t *fb;      //   [n][fbs] fp16 fallback scales
    int32_t fbs;
    const uint8_t *zeros;    // [n][G], or null (implied midpoint zmid)
    uint32_t zmid;
    const int32_t *rowptr;
    const int32_t *col;
    const uint16_t *val;
    const uint16_t *x;
    int64_t ldx, m, n, k, G, gs;
    uint16_t *y;
    int64_t ldy;
    int bits;
    int64_t total_bytes;  // n * k * b / 8
};

// Value of an E4M3 byte (OCP 8-bit float: sign, 4-bit exponent with bias 7, 3-bit mantissa;
// exponent 0 holds the subnormals man * 2^-9; 0x7F and 0xFF are NaN).
float e4m3_value(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15, man = b & 7;
    float v;
    if (e == 15 && man == 7)
        v = __builtin_nanf("");
    else if (e == 0)
        v = (float)man * 0x1p-9f;
    else
        v = ldexpf(1.0f + (float)man * 0.125f, (int)e - 7);
    return (b & 0x80) ? -v : v;
}

// The fp32 scale of group g of row r: the fp16 scale, or with fp8 scales the row factor
// times the byte's E4M3 value (the stored scale, one fp32 product), or for a byte with bit 7
// set the fp16 fallback it indexes (clamped to the row's list; 0 without one).
inline float group_scale(const HostArgs &a, int64_t r, int64_t g)
{
    if (!a.sc8) return half_to_float(a.scales[r * a.G + g]);
    const uint32_t b = a.sc8[r * a.G + g];
    if (b & 0x80) {
        const int j = (int)(b & 0x7F) < a.fbs - 1 ? (int)(b & 0x7F) : a.fbs - 1;
        return j >= 0 ? half_to_float(a.fb[r * a.fbs + j]) : 0.0f;
    }
    return a.rowf[r] * e4m3_value(b);
}

// Outliers of row r added in fp32, then the one fp16 rounding.
void finish_row(const HostArgs &a, int64_t r, const float *acc)
{
    for (int64_t mm = 0; mm < a.m; ++mm) {
        float s = acc[mm];
        if (a.rowptr)
            for (int32_t p = a.rowptr[r]; p < a.rowptr[r + 1]; ++p)
                s = __builtin_fmaf(half_to_float(a.x[mm * a.ldx + a.col[p]]), half_to_float(a.val[p]), s);
        a.y[mm * a.ldy + r] = float_to_half(s);
    }
}

// Portable path: the same fused loop (per group: sum x*q and sum x, then scale), scalar.
void rows_scalar(const HostArgs &a, int64_t r0, int64_t r1)
{
    const int b = a.bits;
    const int64_t rb = a.k * b / 8;
    float acc[8];
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t mm = 0; mm < a.m; ++mm) acc[mm] = 0.f;
        const uint8_t *row = a.w + r * rb;
        for (int64_t g = 0; g < a.G; ++g) {
            const float s = group_scale(a, r, g);
            const float zp = (float)(a.zeros ? a.zeros[r * a.G + g] : a.zmid);
            for (int64_t mm = 0; mm < a.m; ++mm) {
                float sq = 0.f, sx = 0.f;
                for (int64_t kk = g * a.gs; kk < (g + 1) * a.gs; ++kk) {
                    const int64_t bit = kk * b;
                    uint32_t v = row[bit >> 3] | ((uint32_t)(((bit >> 3) + 1 < rb) ? row[(bit >> 3) + 1] : 0) << 8);
                    const uint32_t q = (v >> (bit & 7)) & ((1u << b) - 1);
                    const float xv = half_to_float(a.x[mm * a.ldx + kk]);
                    sq = __builtin_fmaf(xv, (float)q, sq);
                    sx += xv;
                }
                acc[mm] = __builtin_fmaf(s, __builtin_fmaf(-zp, sx, sq), acc[mm]);
            }
        }
        finish_row(a, r, acc);
    }
}

// ---- AVX2 path ---------------------------------------------------------------------------
#define QP_AVX2 __attribute__((target("avx2,fma,f16c")))

// Byte shuffle and shifts that turn a block's b bytes into its 8 codes in 32-bit lanes:
// lane i takes bytes floor(b*i/8) .. +3 and shifts right by (b*i) % 8.
struct Unpacker {
    __m256i shuf, shift, mask;
};

QP_AVX2 Unpacker make_unpacker(int b)
{
    alignas(32) int8_t sh[32];
    alignas(32) int32_t sv[8];
    for (int i = 0; i < 8; ++i) {
        const int byte0 = (b * i) / 8;
        for (int j = 0; j < 4; ++j) {
            const int src = byte0 + j;
            sh[4 * i + j] = (int8_t)(src < 16 ? src : -128);  // 16-byte lanes: both halves see the block
        }
        sv[i] = (b * i) % 8;
    }
    Unpacker u;
    u.shuf = _mm256_load_si256((const __m256i *)sh);
    u.shift = _mm256_load_si256((const __m256i *)sv);
    u.mask = _mm256_set1_epi32((1 << b) - 1);
    return u;
}

QP_AVX2 inline __m256 unpack8(const uint8_t *p, const Unpacker &u)
{
    const __m256i v = _mm256_broadcastsi128_si256(_mm_loadu_si128((const __m128i *)p));
    const __m256i c = _mm256_and_si256(_mm256_srlv_epi32(_mm256_shuffle_epi8(v, u.shuf), u.shift), u.mask);
    return _mm256_cvtepi32_ps(c);
}

// A block read that cannot run past the end of the packed buffer (the last row's tail).
QP_AVX2 inline __m256 unpack8_safe(const HostArgs &a, const uint8_t *p, const Unpacker &u)
{
    alignas(16) uint8_t tmp[16] = {0};
    const int64_t off = p - a.w, left = a.total_bytes - off;
    memcpy(tmp, p, (size_t)(left < 16 ? left : 16));
    return unpack8(tmp, u);
}

QP_AVX2 inline float hsum(__m256 v)
{
    __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    s = _mm_add_ps(s, _mm_movehl_ps(s, s));
    s = _mm_add_ss(s, _mm_movehdup_ps(s));
    return _mm_cvtss_f32(s);
}

// R rows [r0, r0+R) with M activation rows.
template <int R, int M>
QP_AVX2 void rows_avx2_tile(const HostArgs &a, int64_t r0, const Unpacker &u)
{
    const int b = a.bits;
    const int64_t rb = a.k * b / 8, bpg = a.gs / 8;  // bytes per row, blocks per group
    const uint8_t *rows[R];
    bool tail[R];
    for (int i = 0; i < R; ++i) {
        rows[i] = a.w + (r0 + i) * rb;
        tail[i] = (r0 + i) * rb + rb + 16 > a.total_bytes;
    }
    __m256 tot[R][M];
    for (int i = 0; i < R; ++i)
        for (int mm = 0; mm < M; ++mm) tot[i][mm] = _mm256_setzero_ps();
    for (int64_t g = 0; g < a.G; ++g) {
        __m256 acc[R][M], xs[M];
        for (int mm = 0; mm < M; ++mm) xs[mm] = _mm256_setzero_ps();
        for (int i = 0; i < R; ++i)
            for (int mm = 0; mm < M; ++mm) acc[i][mm] = _mm256_setzero_ps();
        for (int64_t j = 0; j < bpg; ++j) {
            const int64_t blk = g * bpg + j, k0 = 8 * blk;
            __m256 xv[M];
            for (int mm = 0; mm < M; ++mm) {
                xv[mm] = _mm256_cvtph_ps(_mm_loadu_si128((const __m128i *)(a.x + mm * a.ldx + k0)));
                xs[mm] = _mm256_add_ps(xs[mm], xv[mm]);
            }
            for (int i = 0; i < R; ++i) {
                const uint8_t *p = rows[i] + blk * b;
                if ((blk & 7) == 0) _mm_prefetch((const char *)(p + 4 * 64), _MM_HINT_T0);
                const __m256 wq = (tail[i] && p + 16 > rows[i] + rb) ? unpack8_safe(a, p, u) : unpack8(p, u);
                for (int mm = 0; mm < M; ++mm) acc[i][mm] = _mm256_fmadd_ps(xv[mm], wq, acc[i][mm]);
            }
        }
        for (int i = 0; i < R; ++i) {
            const int64_t r = r0 + i;
            const float s = group_scale(a, r, g);
            const float zp = (float)(a.zeros ? a.zeros[r * a.G + g] : a.zmid);
            const __m256 vs = _mm256_set1_ps(s), vnz = _mm256_set1_ps(-zp);
            for (int mm = 0; mm < M; ++mm)
                tot[i][mm] = _mm256_fmadd_ps(vs, _mm256_fmadd_ps(vnz, xs[mm], acc[i][mm]), tot[i][mm]);
        }
    }
    for (int i = 0; i < R; ++i) {
        float acc1[8];
        for (int mm = 0; mm < M; ++mm) acc1[mm] = hsum(tot[i][mm]);
        finish_row(a, r0 + i, acc1);
    }
}

template <int M>
QP_AVX2 void rows_avx2_m(const HostArgs &a, int64_t r0, int64_t r1, const Unpacker &u)
{
    constexpr int R = M == 1 ? 4 : M == 2 ? 2 : 1;
    int64_t r = r0;
    for (; r + R <= r1; r += R) rows_avx2_tile<R, M>(a, r, u);
    for (; r < r1; ++r) rows_avx2_tile<1, M>(a, r, u);
}

QP_AVX2 void rows_avx2(const HostArgs &a, int64_t r0, int64_t r1)
{
    const Unpacker u = make_unpacker(a.bits);
    switch (a.m) {
    case 1: rows_avx2_m<1>(a, r0, r1, u); break;
    case 2: rows_avx2_m<2>(a, r0, r1, u); break;
    case 3: rows_avx2_m<3>(a, r0, r1, u); break;
    case 4: rows_avx2_m<4>(a, r0, r1, u); break;
    case 5: rows_avx2_m<5>(a, r0, r1, u); break;
    case 6: rows_avx2_m<6>(a, r0, r1, u); break;
    case 7: rows_avx2_m<7>(a, r0, r1, u); break;
    default: rows_avx2_m<8>(a, r0, r1, u); break;
    }
}

// ---- AVX-512 path (byte permutes of VBMI) -------------------------------------------------
#define QP_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512vbmi,fma,f16c")))
//
// 32 codes (four 8-k blocks, 4b bytes) come from one masked load (it cannot fault past the end
// of the buffer); for each half of 16, one byte permute puts the 4 bytes holding code i into
// 32-bit lane i, one variable left shift moves the code to mantissa bits [23 - b, 23), and one
// ternary-logic op keeps those bits and sets the exponent of 1.0: the lane holds 1 + q / 2^b
// as fp32, exactly, with no integer-to-float conversion.  Per group,
// sum_k x_k (q_k - zp) = 2^b (sum_k x_k (1 + q_k / 2^b)) - (2^b + zp) sum_k x_k.

struct Unpacker512 {
    __m512i perm[2], shl, keep;
};

QP_AVX512 Unpacker512 make_unpacker512(int b)
{
    alignas(64) uint8_t pm[2][64];
    alignas(64) int32_t sv[16];
    for (int h = 0; h < 2; ++h)
        for (int i = 0; i < 16; ++i) {
            const int code = 16 * h + i, byte0 = (b * code) / 8;
            for (int j = 0; j < 4; ++j) pm[h][4 * i + j] = (uint8_t)(byte0 + j < 64 ? byte0 + j : 63);
        }
    for (int i = 0; i < 16; ++i) sv[i] = 23 - b - (b * i) % 8;  // 16 b is a multiple of 8: both halves alike
    Unpacker512 u;
    u.perm[0] = _mm512_load_si512((const void *)pm[0]);
    u.perm[1] = _mm512_load_si512((const void *)pm[1]);
    u.shl = _mm512_load_si512((const void *)sv);
    u.keep = _mm512_set1_epi32(((1 << b) - 1) << (23 - b));
    return u;
}

// R rows [r0, r0+R) with M activation rows.
template <int R, int M>
QP_AVX512 void rows_avx512_tile(const HostArgs &a, int64_t r0, const Unpacker512 &u)
{
    const int b = a.bits, steps = (int)(a.gs / 32);  // 32-code steps per group
    const __mmask64 lm = (__mmask64)((1ull << (4 * b)) - 1);
    const __m512i one = _mm512_set1_epi32(0x3F800000);
    const __m512 vpw = _mm512_set1_ps((float)(1 << b));
    const uint8_t *p = a.w + r0 * (a.k * b / 8);  // the R rows are consecutive: one stream per row
    const int64_t rb = a.k * b / 8;
    const uint8_t *zp8 = a.zeros ? a.zeros + r0 * a.G : nullptr;
    __m512 tot[R][M];
    for (int i = 0; i < R; ++i)
        for (int mm = 0; mm < M; ++mm) tot[i][mm] = _mm512_setzero_ps();
    const uint16_t *xk = a.x;
    for (int64_t g = 0; g < a.G; ++g) {
        __m512 acc[R][M], xs[M];
        for (int mm = 0; mm < M; ++mm) xs[mm] = _mm512_setzero_ps();
        for (int i = 0; i < R; ++i)
            for (int mm = 0; mm < M; ++mm) acc[i][mm] = _mm512_setzero_ps();
        for (int st = 0; st < steps; ++st, xk += 32, p += 4 * b) {
            __m512 xv[2][M];
            for (int mm = 0; mm < M; ++mm)
                for (int h = 0; h < 2; ++h) {
                    xv[h][mm] = _mm512_cvtph_ps(_mm256_loadu_si256((const __m256i *)(xk + mm * a.ldx + 16 * h)));
                    xs[mm] = _mm512_add_ps(xs[mm], xv[h][mm]);
                }
            for (int i = 0; i < R; ++i) {
                _mm_prefetch((const char *)(p + i * rb + 4 * 64), _MM_HINT_T0);
                const __m512i v = _mm512_maskz_loadu_epi8(lm, p + i * rb);
                for (int h = 0; h < 2; ++h) {
                    const __m512i f = _mm512_sllv_epi32(_mm512_permutexvar_epi8(u.perm[h], v), u.shl);
                    const __m512 wq = _mm512_castsi512_ps(_mm512_ternarylogic_epi32(f, u.keep, one, 0xEA));
                    for (int mm = 0; mm < M; ++mm) acc[i][mm] = _mm512_fmadd_ps(xv[h][mm], wq, acc[i][mm]);
                }
            }
        }
        for (int i = 0; i < R; ++i) {
            const float s = group_scale(a, r0 + i, g);
            const float zp = (float)(zp8 ? zp8[i * a.G + g] : a.zmid);
            const __m512 vs = _mm512_set1_ps(s), vnc = _mm512_set1_ps(-((float)(1 << b) + zp));
            for (int mm = 0; mm < M; ++mm)
                tot[i][mm] = _mm512_fmadd_ps(vs, _mm512_fmadd_ps(vpw, acc[i][mm], _mm512_mul_ps(vnc, xs[mm])), tot[i][mm]);
        }
    }
    for (int i = 0; i < R; ++i) {
        float acc1[8];
        for (int mm = 0; mm < M; ++mm) acc1[mm] = _mm512_reduce_add_ps(tot[i][mm]);
        finish_row(a, r0 + i, acc1);
    }
}

template <int M>
QP_AVX512 void rows_avx512_m(const HostArgs &a, int64_t r0, int64_t r1, const Unpacker512 &u)
{
    constexpr int R = M == 1 ? 4 : M == 2 ? 2 : 1;
    int64_t r = r0;
    for (; r + R <= r1; r += R) rows_avx512_tile<R, M>(a, r, u);
    for (; r < r1; ++r) rows_avx512_tile<1, M>(a, r, u);
}

QP_AVX512 void rows_avx512(const HostArgs &a, int64_t r0, int64_t r1)
{
    const Unpacker512 u = make_unpacker512(a.bits);
    switch (a.m) {
    case 1: rows_avx512_m<1>(a, r0, r1, u); break;
    case 2: rows_avx512_m<2>(a, r0, r1, u); break;
    case 3: rows_avx512_m<3>(a, r0, r1, u); break;
    case 4: rows_avx512_m<4>(a, r0, r1, u); break;
    case 5: rows_avx512_m<5>(a, r0, r1, u); break;
    case 6: rows_avx512_m<6>(a, r0, r1, u); break;
    case 7: rows_avx512_m<7>(a, r0, r1, u); break;
    default: rows_avx512_m<8>(a, r0, r1, u); break;
    }
}

// The vector path: AVX-512 (with VBMI) when the CPU has it, else AVX2 with FMA and F16C.
// QPACK_HOST_PORTABLE in the environment selects the portable loop and QPACK_HOST_AVX2 the AVX2
// one (to test them on a host that has more).
enum Path { kPortable, kAvx2, kAvx512 };
Path host_path()
{
    static const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
                             __builtin_cpu_supports("f16c");
    static const bool avx512 = avx2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                               __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512vbmi");
    if (getenv("QPACK_HOST_PORTABLE") || !avx2) return kPortable;
    if (avx512 && !getenv("QPACK_HOST_AVX2")) return kAvx512;
    return kAvx2;
}

int default_threads()
{
#ifdef _OPENMP
    const int p = omp_get_num_procs();
    return p > 2 ? p - 1 : 1;
#else
    return 1;
#endif
}

}  // namespace

extern "C" const char *qlinear_gemv_host_isa(void)
{
    switch (host_path()) {
    case kAvx512: return "avx512vbmi";
    case kAvx2: return "avx2";
    default: return "portable";
    }
}

extern "C" qp_status qlinear_gemv_host(const qp_weight_desc *d, const qp_weight *w, const uint16_t *x, int64_t ldx,
                                       int64_t m, uint16_t *y, int64_t ldy, int32_t threads)
{
    if (!d || !w || !x || !y) return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: NULL argument");
    if (qp_packed_bytes(d) == 0) return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: invalid weight description");
    if (d->layout != QP_LAYOUT_CANONICAL)
        return qp::fail(QP_ERR_UNSUPPORTED, "qlinear_gemv_host reads the canonical layout");
    if (d->zero_mode == QP_ZERO_PACKED)
        return qp::fail(QP_ERR_UNSUPPORTED, "qlinear_gemv_host reads byte or implied zero points");
    if (m < 1 || m > 8) return qp::fail(QP_ERR_UNSUPPORTED, "qlinear_gemv_host handles 1 <= m <= 8 (m=%lld)", (long long)m);
    if (ldx < d->k || ldy < d->n) return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: ldx < k or ldy < n");
    const bool fp8 = d->scale_format == QP_SCALE_FP8;
    if (!w->packed || (!fp8 && !w->scales) || (d->zero_mode == QP_ZERO_STORED && !w->zeros))
        return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: packed/scales/zeros NULL");
    if (fp8) {
        if (!w->scales8 || !w->row_factors) return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: scales8/row_factors NULL");
        if (w->fb_stride < 0 || w->fb_stride > 128 || (w->fb_stride > 0 && !w->fb_scales))
            return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: bad fallback list");
        if (w->nnz != 0 || w->csr_rowptr)
            return qp::fail(QP_ERR_UNSUPPORTED, "qlinear_gemv_host: fp8-scale weights carry no outlier CSR");
    }
    if (w->nnz < 0 || (w->nnz > 0 && (!w->csr_rowptr || !w->csr_col || !w->csr_val)))
        return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: bad outlier CSR");
    if (threads < 0) return qp::fail(QP_ERR_INVALID_ARG, "qlinear_gemv_host: threads < 0");
    HostArgs a;
    a.w = (const uint8_t *)w->packed;
    a.scales = fp8 ? nullptr : w->scales;
    a.sc8 = fp8 ? w->scales8 : nullptr;
    a.rowf = fp8 ? w->row_factors : nullptr;
    a.fb = fp8 && w->fb_stride > 0 ? w->fb_scales : nullptr;
    a.fbs = fp8 ? (int32_t)w->fb_stride : 0;
    a.zeros = d->zero_mode == QP_ZERO_STORED ? w->zeros : nullptr;
    a.zmid = 1u << (d->bits - 1);
    a.rowptr = w->nnz > 0 ? w->csr_rowptr : nullptr;
    a.col = w->csr_col;
    a.val = w->csr_val;
    a.x = x;
    a.ldx = ldx;
    a.m = m;
    a.n = d->n;
    a.k = d->k;
    a.gs = d->group_size;
    a.G = d->k / d->group_size;
    a.y = y;
    a.ldy = ldy;
    a.bits = d->bits;
    a.total_bytes = (int64_t)qp_packed_bytes(d);
    const int nt = threads > 0 ? threads : default_threads();
    const Path path = host_path();
    // Rows in chunks of 16 (a multiple of every row tile), spread over the threads.
    const int64_t chunks = (a.n + 15) / 16;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t c = 0; c < chunks; ++c) {
        const int64_t r0 = 16 * c, r1 = r0 + 16 < a.n ? r0 + 16 : a.n;
        if (path == kAvx512)
            rows_avx512(a, r0, r1);
        else if (path == kAvx2)
            rows_avx2(a, r0, r1);
        else
            rows_scalar(a, r0, r1);
    }
    return QP_OK;
}
