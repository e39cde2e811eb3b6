/*
 * oracle.c - plain, slow CPU reference of the verification hot path.
 *
 * TEST INFRASTRUCTURE ONLY: it is loaded by the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark, never by the product library.
 * It shares no code, header, table or helper with the HIP implementation.
 *
 * Sources, cited by page title and section:
 *  [P1] "GPU-Resident Speculative Decoding for In-Browser LLM Inference with
 *       WebGPU": Design, Small-Batch Verification Kernels; Design, GPU-Resident
 *       Speculation Loop; Implementation.
 *  [P2] "WebGPU for LLM Inference, in depth": A quantised matrix-vector kernel
 *       in WGSL (nibble packing, workgroup tree reduction).
 *  [P3] "Exact Speculative And Assisted Decoding For A Tiny Draft And
 *       Qualified Champion": KV transaction model (commit / rollback).
 *
 * Readings where the pages leave a step open are stated at each function.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 */

float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15);
    uint32_t e = (h >> 10) & 31u;
    uint32_t m = h & 1023u;
    float v;
    if (e == 0) {
        v = (float)m * 5.9604644775390625e-08f; /* m * 2^-24, exact */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        uint32_t bits = ((e - 15u + 127u) << 23) | (m << 13);
        memcpy(&v, &bits, 4);
    }
    return sign ? -v : v;
}

uint16_t orc_f32_to_f16(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t a = b & 0x7fffffffu;
    if (a >= 0x7f800000u) return sign | (a > 0x7f800000u ? 0x7e00u : 0x7c00u);
    if (a >= 0x477ff000u) return sign | 0x7c00u; /* >= 65520 rounds to inf */
    if (a >= 0x38800000u) {                      /* normal fp16 result */
        uint32_t e = (a >> 23) - 127u + 15u;
        uint32_t m = a & 0x7fffffu;
        uint32_t r = (e << 10) | (m >> 13);
        uint32_t rem = m & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r++;
        return sign | (uint16_t)r;
    }
    /* subnormal or zero: value = mant * 2^(E-23), unit of result = 2^-24 */
    int E = (int)(a >> 23) - 127;
    if ((a >> 23) == 0) return sign; /* fp32 denormal: far below 2^-25 */
    uint32_t m = (a & 0x7fffffu) | 0x800000u;
    int s = -(E + 1);                 /* right shift that lands on 2^-24 units */
    if (s >= 32) return sign;
    uint32_t q = m >> s;
    uint32_t rem = m & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return sign | (uint16_t)q;
}

/* ---------------------------------------------------------------- R16 */

/*
 * The fixed reduction order. [P1, Implementation] requires that every matrix
 * multiplication reduce in one fixed order across all token buckets, so that
 * N-token verification gives the bits of N single-token steps; the pages do
 * not print the order. Reading: strided accumulation into a fixed set of
 * partial sums, as in [P2]'s kernel, with 16 partial sums that are then added
 * as a balanced binary tree in index order:
 *   slot s (0..15) starts at +0 and adds v[j] for j = s, s+16, ... in order;
 *   then for w = 1, 2, 4, 8: slot s += slot s+w for every s divisible by 2w,
 *   i.e. ((a0+a1)+(a2+a3)) + ((a4+a5)+(a6+a7)), and so on up to a0.
 */
float orc_r16(const float* v, int64_t n) {
    float a[16];
    for (int s = 0; s < 16; s++) a[s] = 0.0f;
    for (int64_t j = 0; j < n; j++) a[j % 16] = a[j % 16] + v[j];
    for (int w = 1; w < 16; w *= 2)
        for (int s = 0; s < 16; s += 2 * w) a[s] = a[s] + a[s + w];
    return a[0];
}

/* ---------------------------------------------------------------- quant */

/*
 * [P1, Small-Batch Verification Kernels]: activations become 8-bit integers
 * before every matrix multiplication. Readings: one absmax scale per token
 * (not per block of 32); symmetric codes in [-127, 127]; scale = absmax/127
 * and codes round(x * (127/absmax)) to nearest-even, both as single IEEE
 * divisions; an all-zero token has scale 0 and codes 0.
 *
 * Tiny rows. For absmax below about 3.7e-37 the reciprocal 127/absmax
 * overflows to infinity, and every nonzero code would saturate. Reading:
 * when absmax < 2^-64 the row and absmax are first multiplied by 2^64, which
 * is exact, and the codes are round(fl(x * 2^64) * fl(127 / fl(absmax * 2^64))).
 * Wherever 127/absmax is finite this gives exactly the bits of the plain
 * formula: the factor 2^64 commutes with each correctly rounded operation,
 * whose results all stay normal. The scale is absmax/127 either way.
 * Input values must be finite; a NaN or infinity is rejected (-1).
 */
int orc_quantize_act(const float* x, int T, int K, int8_t* xq, float* xs) {
    if (T < 0 || K < 0 || (T > 0 && K > 0 && (!x || !xq || !xs))) return -1;
    for (int64_t i = 0; i < (int64_t)T * K; i++)
        if (!isfinite(x[i])) return -1;
    for (int t = 0; t < T; t++) {
        const float* row = x + (int64_t)t * K;
        float a = 0.0f;
        for (int k = 0; k < K; k++) {
            float v = fabsf(row[k]);
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            xs[t] = 0.0f;
            for (int k = 0; k < K; k++) xq[(int64_t)t * K + k] = 0;
            continue;
        }
        xs[t] = a / 127.0f;
        const float pre = a < 0x1p-64f ? 0x1p64f : 1.0f;
        float inv = 127.0f / (a * pre);
        for (int k = 0; k < K; k++) {
            float r = nearbyintf((row[k] * pre) * inv); /* default mode: nearest-even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[(int64_t)t * K + k] = (int8_t)r;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- linear */

/*
 * Weight format, [P2, quantised matvec]: int4 codes packed eight to a
 * little-endian 32-bit word, code j of the word in bits 4j..4j+3, stored as
 * 0..15 meaning -8..7. Viewed as bytes, byte b of row n holds input 2b in its
 * low nibble and input 2b+1 in its high nibble. [P1, Small-Batch Verification
 * Kernels]: one 16-bit scale per 32 inputs, so group g covers inputs
 * 32g..32g+31, which are the 16 bytes 16g..16g+15 of the row.
 */
static int weight_code(const uint8_t* row, int k) {
    uint8_t b = row[k / 2];
    int u = (k & 1) ? (b >> 4) : (b & 15);
    return u - 8;
}

int orc_group_dots(const uint8_t* wq, const int8_t* xq, int T, int N, int K, int32_t* d) {
    if (T < 0 || N < 0 || K < 0 || K % 32) return -1;
    int G = K / 32;
    for (int t = 0; t < T; t++)
        for (int n = 0; n < N; n++) {
            const uint8_t* row = wq + (int64_t)n * (K / 2);
            for (int g = 0; g < G; g++) {
                int32_t acc = 0;
                for (int kk = 0; kk < 32; kk++) {
                    int k = 32 * g + kk;
                    acc += weight_code(row, k) * (int32_t)xq[(int64_t)t * K + k];
                }
                d[((int64_t)t * N + n) * G + g] = acc;
            }
        }
    return 0;
}

/*
 * One output y[t][n] ([P1, Small-Batch Verification Kernels]: integer dot
 * products per 32-input block, then the block's 16-bit scale):
 *   d_g = sum over the group of code * xq, exact in int32;
 *   p_g = f32(scale_g) * f32(d_g), one rounding;
 *   y   = xs[t] * R16(p_0 .. p_{G-1}), one rounding.
 */
static float linear_one(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                        const float* xs, int t, int n, int K, float* p) {
    int G = K / 32;
    const uint8_t* row = wq + (int64_t)n * (K / 2);
    const int8_t* xr = xq + (int64_t)t * K;
    for (int g = 0; g < G; g++) {
        int32_t d = 0;
        for (int kk = 0; kk < 32; kk++) d += weight_code(row, 32 * g + kk) * (int32_t)xr[32 * g + kk];
        p[g] = orc_f16_to_f32(ws[(int64_t)n * G + g]) * (float)d;
    }
    return xs[t] * orc_r16(p, G);
}

int orc_w4a8_linear(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                    const float* xs, float* y, int T, int N, int K) {
    if (T < 0 || N < 0 || K < 32 || K % 32) return -1;
    float* p = (float*)malloc(sizeof(float) * (size_t)(K / 32));
    if (!p) return -1;
    for (int t = 0; t < T; t++)
        for (int n = 0; n < N; n++) y[(int64_t)t * N + n] = linear_one(wq, ws, xq, xs, t, n, K, p);
    free(p);
    return 0;
}

/*
 * Per-block activation scales, the format of [P1, Small-Batch Verification
 * Kernels] (activations quantised to 8-bit integers per block of 32 values).
 * Readings: the block is a weight group (inputs 32g..32g+31); its scale is
 * absmax/127 and its codes round(x * (127/absmax)) to nearest-even, as for a
 * token above; an all-zero block has scale 0 and codes 0. xs is [T][K/32].
 */
int orc_quantize_act_blocks(const float* x, int T, int K, int8_t* xq, float* xs) {
    if (T < 0 || K < 0 || K % 32 || (T > 0 && K > 0 && (!x || !xq || !xs))) return -1;
    const int G = K / 32;
    for (int t = 0; t < T; t++)
        for (int g = 0; g < G; g++)
            if (orc_quantize_act(x + (int64_t)t * K + 32 * g, 1, 32, xq + (int64_t)t * K + 32 * g,
                                 xs + (int64_t)t * G + g) != 0)
                return -1;
    return 0;
}

/*
 * W4A8 linear with per-block activation scales. Reading: each group's two
 * scales combine first, then meet the exact integer dot, and the products
 * are summed in the fixed order with no trailing scale:
 *   s_g = f32(scale_g) * xs[t][g],  one rounding;
 *   p_g = s_g * f32(d_g),            one rounding;
 *   y   = R16(p_0 .. p_{G-1}).
 */
int orc_w4a8_linear_blocks(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                           const float* xs, float* y, int T, int N, int K) {
    if (T < 0 || N < 0 || K < 32 || K % 32) return -1;
    const int G = K / 32;
    float* p = (float*)malloc(sizeof(float) * (size_t)G);
    if (!p) return -1;
    for (int t = 0; t < T; t++)
        for (int n = 0; n < N; n++) {
            const uint8_t* row = wq + (int64_t)n * (K / 2);
            const int8_t* xr = xq + (int64_t)t * K;
            for (int g = 0; g < G; g++) {
                int32_t d = 0;
                for (int kk = 0; kk < 32; kk++) d += weight_code(row, 32 * g + kk) * (int32_t)xr[32 * g + kk];
                const float s = orc_f16_to_f32(ws[(int64_t)n * G + g]) * xs[(int64_t)t * G + g];
                p[g] = s * (float)d;
            }
            y[(int64_t)t * N + n] = orc_r16(p, G);
        }
    free(p);
    return 0;
}

int orc_w4a8_linear_rows(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                         const float* xs, float* y, int T, int N, int K,
                         const int32_t* rows, int nrows) {
    if (T < 0 || N < 0 || K < 32 || K % 32 || nrows < 0) return -1;
    for (int r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= N) return -1;
    float* p = (float*)malloc(sizeof(float) * (size_t)(K / 32));
    if (!p) return -1;
    for (int t = 0; t < T; t++)
        for (int r = 0; r < nrows; r++)
            y[(int64_t)t * nrows + r] = linear_one(wq, ws, xq, xs, t, rows[r], K, p);
    free(p);
    return 0;
}

/* ---------------------------------------------------------------- argmax */

/*
 * Greedy prediction per tree node ([P1, GPU-Resident Speculation Loop]).
 * Reading: the lowest index among equal maxima; comparison with IEEE '>', so
 * -0 and +0 are equal. NaN inputs are outside the contract.
 */
int orc_argmax(const float* logits, int N, int64_t V, int32_t* out) {
    if (N < 0 || V <= 0) return -1;
    for (int i = 0; i < N; i++) {
        const float* r = logits + (int64_t)i * V;
        int64_t best = 0;
        for (int64_t v = 1; v < V; v++)
            if (r[v] > r[best]) best = v;
        out[i] = (int32_t)best;
    }
    return 0;
}

/* ---------------------------------------------------------------- accept */

/*
 * [P1, GPU-Resident Speculation Loop]: node 0 is the token of the previous
 * step, nodes 1..N-1 the draft tree; acceptance follows, from the root, the
 * child whose token equals its parent's greedy prediction; the step commits
 * the accepted draft nodes plus the prediction after the last of them.
 * Reading for duplicate sibling tokens: a node is accepted when its parent is
 * accepted and its token equals the parent's prediction; the winner is the
 * deepest accepted node, the lowest index among equally deep ones.
 * Trees must be topologically ordered: parent[0] = -1, 0 <= parent[i] < i.
 */
int orc_tree_accept(const int32_t* parent, const int32_t* token, const int32_t* amax,
                    int N, int32_t* path, int32_t* bonus) {
    if (N < 1 || N > 64 || parent[0] != -1) return -1;
    int acc[64], depth[64];
    acc[0] = 1;
    depth[0] = 0;
    for (int i = 1; i < N; i++) {
        if (parent[i] < 0 || parent[i] >= i) return -1;
        acc[i] = acc[parent[i]] && token[i] == amax[parent[i]];
        depth[i] = depth[parent[i]] + 1;
    }
    int w = 0;
    for (int i = 1; i < N; i++)
        if (acc[i] && depth[i] > depth[w]) w = i;
    int m = depth[w];
    for (int i = w, j = m; j >= 0; j--) {
        path[j] = i;
        i = parent[i];
    }
    *bonus = amax[w];
    return m;
}

/* ---------------------------------------------------------------- compact */

/*
 * [P1, GPU-Resident Speculation Loop]: compaction moves the keys and values
 * of the accepted path into place. [P3, KV transaction model]: rows past the
 * committed pointer are dead, rollback is a pointer move. Tree node i was
 * written at physical row L+i; accepted node path[j] (depth j) moves to row
 * L+j, j = 1..m in increasing order, which is safe in place because
 * path[j] >= j.
 */
int orc_kv_compact(uint16_t* cache, int layers, int heads, int cap, int hd,
                   int L, const int32_t* path, int m) {
    if (layers < 0 || heads < 0 || cap < 0 || hd < 0 || L < 0 || m < 0) return -1;
    for (int j = 1; j <= m; j++)
        if (path[j] < j || L + path[j] >= cap) return -1;
    for (int l = 0; l < layers; l++)
        for (int h = 0; h < heads; h++) {
            uint16_t* base = cache + ((int64_t)l * heads + h) * (int64_t)cap * hd;
            for (int j = 1; j <= m; j++)
                memmove(base + (int64_t)(L + j) * hd, base + (int64_t)(L + path[j]) * hd,
                        sizeof(uint16_t) * (size_t)hd);
        }
    return 0;
}
