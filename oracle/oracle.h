/*
 * oracle.h - plain, slow CPU reference of the verification hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library includes this
 * header, links this code or calls it; only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load liboracle.so.
 *
 * Every floating-point operation is one IEEE-754 binary32 operation rounded
 * to nearest-even, in the order the comments state. The file is compiled with
 * -O2 -ffp-contract=off -fno-fast-math and no -march, so no FMA is formed
 * and nothing is reassociated. Denormals are kept.
 *
 * Status codes: 0 on success, -1 for an invalid argument.
 */
#ifndef SPECV_ORACLE_H
#define SPECV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* fp16 <-> fp32. Widening is exact; narrowing rounds to nearest-even with
 * overflow to infinity and gradual underflow. */
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float x);

/* The fixed 16-slot summation order used by every fp32 sum of the path. */
float orc_r16(const float* v, int64_t n);

/* Per-token absmax int8 quantisation of x [T][K] -> xq [T][K], xs [T]. */
int orc_quantize_act(const float* x, int T, int K, int8_t* xq, float* xs);

/* Exact int32 dot of each 32-input group: d [T][N][K/32]. */
int orc_group_dots(const uint8_t* wq, const int8_t* xq, int T, int N, int K, int32_t* d);

/* W4A8 linear: y [T][N] from nibbles wq [N][K/2], fp16 scales ws [N][K/32],
 * codes xq [T][K] and token scales xs [T]. */
int orc_w4a8_linear(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                    const float* xs, float* y, int T, int N, int K);

/* Same, for a list of output rows only: y [T][nrows] holds rows[r]. */
int orc_w4a8_linear_rows(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                         const float* xs, float* y, int T, int N, int K,
                         const int32_t* rows, int nrows);

/* Per-block variants: one activation scale per token and 32-input block,
 * xs [T][K/32]; the linear sums fl(fl(scale * xs) * d) in the fixed order. */
int orc_quantize_act_blocks(const float* x, int T, int K, int8_t* xq, float* xs);
int orc_w4a8_linear_blocks(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                           const float* xs, float* y, int T, int N, int K);

/* Lowest index of the maximum of each row of logits [N][V]. */
int orc_argmax(const float* logits, int N, int64_t V, int32_t* out);

/* Greedy tree acceptance. Returns the accepted depth m >= 0 and fills
 * path[0..m] and *bonus, or -1 for a malformed tree. */
int orc_tree_accept(const int32_t* parent, const int32_t* token, const int32_t* amax,
                    int N, int32_t* path, int32_t* bonus);

/* In-place compaction of one cache [layers][heads][cap][hd] (fp16 bits):
 * row L+path[j] moves to row L+j for j = 1..m. */
int orc_kv_compact(uint16_t* cache, int layers, int heads, int cap, int hd,
                   int L, const int32_t* path, int m);

/* Context-mixing drafter (drafter.c): the next tree from the token stream
 * s[0..n) whose last token is the pending root. weight[l] (l = 1..8, in
 * [1, 2^24]) is the weight of a candidate with match length l. Returns the node
 * count (1..width) and fills parent/token [width] and *best_match, or -1. */
int orc_cm_draft(const int32_t* s, int n, int max_order, int cands, int depth, const uint32_t* weight,
                 int width, int32_t* parent, int32_t* token, int32_t* best_match);

#ifdef __cplusplus
}
#endif

/* ------------------------------------------------------------------ forward
 * Tree-masked forward of a small-batch verification step and the
 * device-resident speculation window, for a Qwen2.5-shaped decoder. All
 * weights use the W4A8 format above with row-major scales [rows][K/32]. */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab, max_pos;
    float eps;
    /* per layer (arrays of n_layers host pointers) */
    const uint8_t* const* wq; const uint16_t* const* sq;  /* [nh*hd][H]   */
    const uint8_t* const* wk; const uint16_t* const* sk;  /* [nkv*hd][H]  */
    const uint8_t* const* wv; const uint16_t* const* sv;  /* [nkv*hd][H]  */
    const uint8_t* const* wo; const uint16_t* const* so;  /* [H][nh*hd]   */
    const uint8_t* const* wg; const uint16_t* const* sg;  /* [I][H]       */
    const uint8_t* const* wu; const uint16_t* const* su;  /* [I][H]       */
    const uint8_t* const* wd; const uint16_t* const* sd;  /* [H][I]       */
    const float* const* norm_attn; const float* const* norm_mlp;  /* [H] */
    const float* norm_final;                                      /* [H] */
    const uint8_t* wlm; const uint16_t* slm;                      /* [V][H] */
    const float* rope_cos; const float* rope_sin;                 /* [max_pos][hd/2] */
} orc_model;

float orc_det_exp(float x);
float orc_silu(float g);
void orc_rmsnorm(const float* x, const float* w, int H, float eps, float* y);
int orc_rope_table(float* cos_t, float* sin_t, int max_pos, int head_dim, double theta);

/* Chunked attention of one query head (scores scaled by 1/sqrt(hd)) over the KV rows
 * `rows` (logical order) of one head plane [..][hd] (fp16 bits). */
int orc_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int hd, const int* rows,
                  int len, float* out);

/* One forward pass over a tree of N nodes whose root sits at committed
 * length L: writes K/V rows L+i of every layer and logits [N][V]. */
int orc_forward(const orc_model* m, uint16_t* kc, uint16_t* vc, int cap, int L, int N,
                const int32_t* parent, const int32_t* token, float* logits);

/* A full verification step: forward, argmax, acceptance and compaction.
 * *L advances by m+1; returns m (>= 0) and fills path[0..m], amax[0..N),
 * *bonus; or -1 on bad arguments. logits may be NULL. */
int orc_tree_step(const orc_model* m, uint16_t* kc, uint16_t* vc, int cap, int* L, int N,
                  const int32_t* parent, const int32_t* token, float* logits, int32_t* amax,
                  int32_t* path, int32_t* bonus);

/* Synthetic drafter of the window: the tree for one step. */
int orc_draft_tree(int width, int L, int32_t root_token, const int32_t* greedy, int stream_len,
                   const uint32_t* draws, uint32_t threshold, int vocab, int32_t* parent,
                   int32_t* token, int* best_match);

#ifdef __cplusplus
}
#endif
#endif
