// Internal interfaces between the library's sources (not part of the ABI).
#pragma once

#include <algorithm>

#include "common.h"

namespace specv {

// Byte offsets of one step's buffers inside the caller's workspace.
struct StepLayout {
    size_t h, delta, xq, xs, qkv, qrot, attn, gu, logits, argmax_part, tree, tinfo, wcounter, linear;
    size_t linear_bytes, total;
    int nchunk_max;
};

StepLayout step_layout(const specv_model* m, int n_max);
int validate_model(const specv_model* m);

// W4A8 linear on validated arguments; y may be null when amax is set. The
// argmax epilogue (amax: [T][chunks] partials) needs linear_argmax_supported.
int linear_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, Best* amax,
                   int T, int N, int K, void* workspace, hipStream_t s);
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

}  // namespace specv
