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

// Argmax per node and tree acceptance. When wcounter is not null the step's
// statistics go to stats[*wcounter] and the counter advances.
int enqueue_argmax_accept(const float* logits, int64_t V, int n_max, const int32_t* parent,
                          const int32_t* token, int32_t* argmax, int32_t* path, specv_ctrl* ctrl,
                          specv_step_stats* stats, int32_t* wcounter, int32_t* ring, int32_t ring_cap,
                          void* partials, hipStream_t s);

int enqueue_forward(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                    specv_ctrl* ctrl, char* ws, const StepLayout& lay, hipStream_t s);

int enqueue_step(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                 int32_t* argmax, int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* wcounter,
                 int32_t* ring, int32_t ring_cap, char* ws, const StepLayout& lay, hipStream_t s);

}  // namespace specv
