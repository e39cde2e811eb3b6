// Internal interfaces between the library's sources (not part of the ABI).
#pragma once

#include <algorithm>

#include "common.h"

namespace specv {

// Byte offsets of one step's buffers inside the caller's workspace.
struct StepLayout {
    size_t h, h2, delta, xq, xs, qkv, attn, gu, logits, argmax_part, tree, tinfo, wcounter, arrivals, linear;
    size_t linear_bytes, total;
    int nchunk_max;
};

StepLayout step_layout(const specv_model* m, int n_max);

// Activation rows a linear can produce itself, in its prologue, instead of
// reading codes a row kernel wrote: every workgroup computes the rows of all
// tokens with the row kernel's arithmetic (so the codes are the same bits).
//   kProdNorm: x = a (+ b), written to h_out by workgroup 0 when h_out is
//              set; RMSNorm with weight w and eps; per-token quantisation.
//   kProdRows: the rows a[t][k] as they are (the SiLU-gated rows the
//              gate_up epilogue wrote); per-token quantisation.
// Tokens at or past ctrl->n_nodes, or all tokens once ctrl->done is set,
// quantise to zero.
enum { kProdNone = 0, kProdNorm = 1, kProdRows = 2 };
// What the linear writes: its outputs y[t][n] (kEpiPlain), or, for a matrix
// whose rows alternate in blocks of 8 gate rows and 8 up rows (16-row tile
// b: gate rows 8b..8b+7, then up rows 8b..8b+7), z[t][i] = silu(g) * u with
// g and u the outputs of gate row i and up row i (kEpiSiluPairs; y is
// [T][N/2]).
enum { kEpiPlain = 0, kEpiSiluPairs = 1 };
struct ProdArgs {
    const float* a;
    const float* b;
    const float* w;
    float* h_out;
    float eps;
    int pad;
    const specv_ctrl* ctrl;
    int epi;
};

// W4A8 linear whose activations the kernel produces (T <= 16, per-token
// scales, activations kept in LDS). Returns SPECV_E_SHAPE, enqueueing
// nothing, when the shape does not allow it.
int linear_enqueue_fused(int prod, const ProdArgs& pa, const uint8_t* wq, const uint16_t* ws, float* y, Best* amax,
                         int T, int N, int K, hipStream_t s);
bool linear_fused_supported(int prod, int T, int K);
int validate_model(const specv_model* m);

// W4A8 linear on validated arguments; y may be null when amax is set. The
// argmax epilogue (amax: [T][chunks] partials) needs linear_argmax_supported.
int linear_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, Best* amax,
                   int T, int N, int K, void* workspace, hipStream_t s, int epi = kEpiPlain);
// The 32-token bucket with dense matrix products (17..32 tokens, per-token
// scales, at most 10 x 16 groups per row), in csrc/linear_dense.hip.
bool linear_dense_supported(int T, int K);
// The events set by specv_time_next_linear for the next linear launch, if
// any (cleared by this call).
bool take_linear_timing(hipEvent_t* start, hipEvent_t* stop);
int linear_dense_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, int T,
                         int N, int K, hipStream_t s);
bool linear_argmax_supported(int T, int N, int K);
int linear_argmax_chunks(int T, int N, int K);

// Tree acceptance from argmax partials ([n_max][chunks]) or, when amax_in is
// set, from the argmax of each node; argmax_out is nullable.
int enqueue_accept(const Best* part, int chunks, const int32_t* amax_in, int n_max, const int32_t* parent,
                   const int32_t* token, int32_t* argmax_out, int32_t* path, specv_ctrl* ctrl,
                   specv_step_stats* stats, int32_t* wcounter, int32_t* ring, int32_t ring_cap, hipStream_t s);

// Argmax per node and tree acceptance. When wcounter is not null the step's
// statistics go to stats[*wcounter] and the counter advances.
int enqueue_argmax_accept(const float* logits, int64_t V, int n_max, const int32_t* parent,
                          const int32_t* token, int32_t* argmax, int32_t* path, specv_ctrl* ctrl,
                          specv_step_stats* stats, int32_t* wcounter, int32_t* ring, int32_t ring_cap,
                          void* partials, hipStream_t s);

int enqueue_forward(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                    Best* amax, specv_ctrl* ctrl, char* ws, const StepLayout& lay, hipStream_t s);

// One step: forward, acceptance, compaction. logits may be null (not wanted).

int enqueue_step(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                 int32_t* argmax, int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* wcounter,
                 int32_t* ring, int32_t ring_cap, char* ws, const StepLayout& lay, hipStream_t s);

// Context-mixing drafter. With ctrl set, the stream is the ring (length
// committed_len + 1) and the tree's size and best match go to ctrl and
// stats[*wcounter]; otherwise the stream has n_given tokens and they go to
// n_nodes_out and best_match_out. cap: stream capacity (scan grid size).
bool cm_params_ok(const specv_cm_params* p);
size_t cm_workspace_bytes(int cap, const specv_cm_params* p);
int enqueue_cm_draft(const int32_t* s, int n_given, int cap, specv_ctrl* ctrl, const specv_cm_params* p, int width,
                     int32_t* parent, int32_t* token, int32_t* n_nodes_out, int32_t* best_match_out,
                     specv_step_stats* stats, const int32_t* wcounter, void* workspace, hipStream_t st);

}  // namespace specv
