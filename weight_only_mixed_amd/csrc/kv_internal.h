// Internal declarations of the quantized KV cache (kvattn.hip, api.hip).
#pragma once

#include "qp_internal.h"

namespace qp {

// Quantized KV cache (kvattn.hip).
struct KvQuantArgs {
    const uint16_t *x;     // [rows][ldx] fp16 head vectors
    int64_t ldx;
    const int64_t *slots;  // [rows] cache row of each input row
    int64_t rows;
    int64_t total_rows;    // batch * kv_heads * capacity
    int64_t cap;           // capacity (tokens per sequence and kv head)
    uint8_t *codes;
    float *scales;
};
hipError_t launch_kv_quantize(int bits, int which, int g, const KvQuantArgs &a, hipStream_t st);

struct KvAttnArgs {
    const uint16_t *q;     // [batch][hq][128]
    const uint8_t *kc;
    const float *ks;
    const uint8_t *vc;
    const float *vs;
    const int32_t *lens;   // [batch]
    uint16_t *o;           // [batch][hq][128]
    float *part_o;         // [batch*hq][nsplit][128] (nsplit > 1)
    float *part_ml;        // [batch*hq][nsplit][2]: chunk maximum (base 2) and weight sum
    int64_t cap;
    int32_t hq, hkv, grp, nsplit, chunk;
    float c;               // softmax scale times log2(e)
};
hipError_t launch_kv_attn(int kb, int vb, int kg, int vg, int64_t batch, const KvAttnArgs &a, hipStream_t st);
void kv_split(int64_t batch, int64_t hkv, int64_t cap, int32_t *nsplit, int32_t *chunk);

}  // namespace qp
