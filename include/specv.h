/*
 * specv.h - C ABI of the deterministic small-batch verification library
 * (libspecv.so, HIP for AMD Instinct MI355X / gfx950).
 *
 * The operations follow "GPU-Resident Speculative Decoding for In-Browser LLM
 * Inference with WebGPU" (cited below as [P1] with its section), the packing
 * of "WebGPU for LLM Inference, in depth" ([P2], quantised matvec kernel) and
 * the KV transaction model of "Exact Speculative And Assisted Decoding For A
 * Tiny Draft And Qualified Champion" ([P3]).
 *
 * Conventions shared by every call:
 *  - Pointers are device memory unless marked "host". The caller owns and
 *    allocates every buffer; the library allocates nothing.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call validates its arguments on the host, enqueues its kernels on
 *    `stream` and returns without synchronising. Device faults surface at the
 *    caller's next synchronisation.
 *  - On invalid arguments a call returns a negative status and enqueues
 *    nothing. No call aborts, throws or falls back to another code path.
 *  - Tensors are dense row-major (C order) unless stated otherwise.
 *  - Results are deterministic: the same inputs give the same bits on every
 *    run, launch shape and token count.
 */
#ifndef SPECV_H
#define SPECV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SPECV_OK = 0,
    SPECV_E_INVAL = -1,     /* null pointer, negative size, bad enum value  */
    SPECV_E_SHAPE = -2,     /* size outside the supported range             */
    SPECV_E_ALIGN = -3,     /* pointer not aligned as the call requires     */
    SPECV_E_HIP = -4,       /* the HIP runtime refused a launch             */
    SPECV_E_WORKSPACE = -5  /* workspace missing or smaller than required   */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* specv_status_string(int status);

/*
 * Device-resident control state, 32 bytes ([P1], GPU-Resident Speculation
 * Loop: the committed KV length, the number of valid nodes, the context
 * length and a termination flag live in a small buffer every kernel reads at
 * run time). Kernels read these fields from device memory when they run, so a
 * sequence of steps can be enqueued without host decisions in between.
 *   committed_len  KV rows [0, committed_len) are committed.
 *   n_nodes        valid tree nodes of the current step (1..16).
 *   ctx_len        context limit: a step that leaves committed_len + n_nodes
 *                  > ctx_len sets done, so the next tree still fits.
 *   done           non-zero: every step kernel returns without effect.
 *   accept_len     m, accepted draft nodes of the last step (0 if it was a
 *                  no-op).
 *   root_token     token of node 0 of the next step (the last step's bonus).
 *   step           steps committed so far.
 *   ring_head      tokens emitted so far (next ring slot = ring_head % cap).
 */
typedef struct {
    int32_t committed_len;
    int32_t n_nodes;
    int32_t ctx_len;
    int32_t done;
    int32_t accept_len;
    int32_t root_token;
    int32_t step;
    int32_t ring_head;
} specv_ctrl;

/* Per-step statistics, 12 bytes ([P1], GPU-Resident Speculation Loop; the
 * controller of Feedback Control of Speculation Width reads the accepted
 * count and the drafter's best match length). */
typedef struct {
    int32_t accepted;    /* m of the step, -1 if the step was a no-op */
    int32_t best_match;  /* drafter's best candidate length (0 if unknown) */
    int32_t width;       /* n_nodes of the step */
} specv_step_stats;

/*
 * Per-token int8 activation quantisation ([P1], Small-Batch Verification
 * Kernels: activations become 8-bit integers before every matrix
 * multiplication; here with one absmax scale per token).
 *   x   fp32 [T][K]      input activations (finite values).
 *   xq  int8 [T][K]      codes: round-to-nearest-even of x * (127/absmax),
 *                        in [-127, 127].
 *   xs  fp32 [T]         scale absmax/127 (0 for an all-zero token, whose
 *                        codes are 0).
 * T in [0, 2^20] rows (one workgroup each), K in [1, 2^24]. T == 0 enqueues
 * nothing.
 * Alignment: x 4 bytes; xq and xs any.
 */
int w4a8_quantize_act(const float* x, int32_t T, int32_t K, int8_t* xq, float* xs,
                      void* stream);

/*
 * Per-block int8 activation quantisation ([P1], Small-Batch Verification
 * Kernels: each token's activations are quantised per block of 32 values):
 * as w4a8_quantize_act, with one absmax scale per token and 32-input block.
 *   x   fp32 [T][K]      input activations (finite values).
 *   xq  int8 [T][K]      codes: round-to-nearest-even of x * (127/absmax of
 *                        the block), in [-127, 127].
 *   xs  fp32 [T][K/32]   scale absmax/127 per block (0 for an all-zero block,
 *                        whose codes are 0).
 * T in [0, 2^20], K a multiple of 32 in [32, 2^24], T*K < 2^31. T == 0
 * enqueues nothing.
 * Alignment: x 16 bytes, xq and xs 4.
 */
int w4a8_quantize_act_blocks(const float* x, int32_t T, int32_t K, int8_t* xq, float* xs, void* stream);

/*
 * Packed tile layout of the W4A8 weights, made once when a model is loaded.
 * The interchange format is the one [P2] (A quantised matrix-vector kernel
 * in WGSL) packs: nibbles row-major, byte b of row n holding input 2b in the
 * low nibble and input 2b+1 in the high nibble, each stored as u = q + 8,
 * and one fp16 scale per row and group of 32 inputs. The linear kernels
 * read 16-row tiles group by group, so the packed layout stores each tile's
 * bytes in that order and every wavefront load is one contiguous kilobyte:
 *   wq  uint8 [N][K/2]    interchange nibbles (device memory).
 *   ws  uint16 [N][K/32]  interchange fp16 scale bits (device memory).
 *   wp  uint8,  w4a8_packed_weight_bytes(N, K) bytes: the 16 bytes of row
 *       16t + r, group g (inputs 32g .. 32g + 31) at byte offset
 *       ((t*G + g)*16 + r)*16, with G = K/32 and t < ceil(N/16).
 *   sp  uint16, w4a8_packed_scale_bytes(N, K) bytes: the scale of row
 *       16t + r, group g at element (t*G + g)*16 + r.
 * Rows from N up to the next multiple of 16 are written as zeros. The call
 * only moves bytes; it enqueues one kernel on `stream`.
 * N in [1, 2^24], K a multiple of 32 in [32, 2^20], packed weights
 * < 2^31 bytes. Alignment: wq, wp 16 bytes; ws, sp 2.
 */
size_t w4a8_packed_weight_bytes(int32_t N, int32_t K);
size_t w4a8_packed_scale_bytes(int32_t N, int32_t K);
int w4a8_pack_weights(const uint8_t* wq, const uint16_t* ws, int32_t N, int32_t K, uint8_t* wp, uint16_t* sp,
                      void* stream);

/*
 * The weights must be in the packed tile layout of w4a8_pack_weights: the
 * interchange layout ([N][K/2] nibbles, [N][K/32] scales) passed here gives
 * wrong outputs with status SPECV_OK, since a layout cannot be checked.
 *
 * W4A8 linear for T = 1..32 tokens ([P1], Small-Batch Verification Kernels
 * and Implementation; packing of [P2]):
 *   y[t][n] = xs[t] * R16_g( f32(ws[g][n]) * f32(d[t][n][g]) ),
 *   d[t][n][g] = sum_{k in group g} (u(n,k) - 8) * xq[t][k]   (exact int32),
 * where R16 is the fixed 16-slot order: slot s accumulates the groups
 * g = s, s+16, ... in increasing g starting from +0, then the 16 slots are
 * added as a binary tree in index order (slot s += slot s+w for s divisible
 * by 2w, w = 1, 2, 4, 8). The order does not depend on T, so row t of a
 * T-token call equals a 1-token call on token t bit for bit.
 *   wq, ws  the weights and scales in the packed tile layout of
 *           w4a8_pack_weights (codes u(n,k) = q + 8, one fp16 scale per 32
 *           inputs).
 *   xq  int8 [T][K], xs fp32 [T]   from w4a8_quantize_act.
 *   y   fp32 [T][N]
 *   workspace  unused (w4a8_linear_workspace returns 0 for every shape);
 *              any value, NULL included, is accepted.
 * T in [1, 32] (the buckets of [P1] are 1, 2, 4, 8, 16 and 32 tokens; 17..31
 * run in the 32-token kernel), N in [0, 2^24], K a multiple of 32 in
 * [32, 2^20], w4a8_packed_weight_bytes(N, K) < 2^31. N == 0 enqueues
 * nothing. The fp16 scales must be finite for T in 8..32: those buckets
 * form each scaled product as one fused multiply-add, exact for every
 * finite scale, and an infinite or NaN scale gives NaN instead of +-inf
 * (below 8 tokens every fp16 scale gives the IEEE product).
 * Alignment: wq and xq 16 bytes, ws 2, xs and y 4.
 */
size_t w4a8_linear_workspace(int32_t T, int32_t N, int32_t K);
int w4a8_linear_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                  float* y, int32_t T, int32_t N, int32_t K, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * W4A8 linear with per-block activation scales ([P1], Small-Batch
 * Verification Kernels: activations quantised per block of 32 values, each
 * block meeting one weight group), in the same fixed order:
 *   y[t][n] = R16_g( ( f32(ws[g][n]) * xs[t][g] ) * f32(d[t][n][g]) ),
 * each product rounded once, the two scales combined first; d and R16 as in
 * w4a8_linear_T. Row t of a T-token call equals a 1-token call on token t.
 *   xq  int8 [T][K], xs fp32 [T][K/32]   from w4a8_quantize_act_blocks.
 * Other arguments, ranges and alignments as w4a8_linear_T (no workspace).
 */
int w4a8_linear_blocks_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                         float* y, int32_t T, int32_t N, int32_t K, void* stream);

/*
 * W4A8 linear with a fused argmax epilogue ([P1], GPU-Resident Speculation
 * Loop: the greedy prediction of each tree node; here fused into the lm_head
 * as the ranked next step of the hot path). Computes the same y as
 * w4a8_linear_T and argmax[t] = the lowest n with y[t][n] = max_n y[t][n]
 * (IEEE comparison, -0 == +0; NaN outputs are a precondition violation).
 * Each workgroup reduces its rows to one (value, index) pair per token, so
 * the outputs need not be written:
 *   y        nullable fp32 [T][N]: written only when non-NULL.
 *   argmax   int32 [T] out.
 *   workspace  w4a8_linear_argmax_workspace(T, N, K) bytes, 8-byte aligned,
 *              no initialisation needed (the per-workgroup pairs).
 * Shapes as w4a8_linear_T with N >= 1, limited to those whose staged
 * activations fit one workgroup (w4a8_linear_argmax_workspace returns 0 and
 * the call SPECV_E_SHAPE otherwise; T * K <= 37888 always fits).
 */
size_t w4a8_linear_argmax_workspace(int32_t T, int32_t N, int32_t K);
int w4a8_linear_argmax_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                         float* y, int32_t* argmax, int32_t T, int32_t N, int32_t K, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * w4a8_linear_argmax_T without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workgroups' (value, row) pairs go to
 * a static device array of the library (128 KiB per device, held until the
 * process ends), so the call allocates nothing. Same arguments, results and
 * errors as w4a8_linear_argmax_T; shapes whose pairs need more than 128 KiB
 * (T * chunks * 8 bytes; chunks is at most two per compute unit) return
 * SPECV_E_WORKSPACE and enqueue nothing. Every call on one device shares that
 * array: calls that overlap on one device (two streams, or two threads)
 * race and give undefined predictions; calls on one stream are ordered.
 */
int w4a8_linear_argmax_T_noalloc(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                                 const float* xs, float* y, int32_t* argmax, int32_t T, int32_t N,
                                 int32_t K, void* stream);

/*
 * Timing diagnostic (not part of the computation): the next w4a8_linear_T
 * launch made by the calling host thread records `start_event` and
 * `stop_event` (hipEvent_t created with timing) at the beginning and end of
 * its kernel (hipExtLaunchKernel), so a benchmark can time one kernel without
 * the queue's event packets around it. Both NULL cancels a pending request;
 * exactly one NULL returns SPECV_E_INVAL. A call that returns an error
 * before launching leaves the request pending.
 */
int specv_time_next_linear(void* start_event, void* stop_event);

/*
 * Measurement diagnostic (not part of the computation): reads `bytes` bytes
 * at p (device memory, 16-byte aligned, bytes a multiple of 16) with `grid`
 * workgroups of 256 threads, each thread keeping four 16-byte loads in
 * flight, and does nothing with them (sink, 4 bytes of device memory, is
 * written only if the folded bytes equal a fixed sentinel). It gives the
 * rate at which the same bytes stream with no arithmetic; bytes == 0 is an
 * empty launch, for the per-launch cost of the queue. grid in [1, 65536].
 * Returns SPECV_E_INVAL or SPECV_E_ALIGN on bad arguments, enqueueing
 * nothing.
 */
int specv_stream_read(const void* p, size_t bytes, uint32_t* sink, int32_t grid, void* stream);

/*
 * Greedy argmax per tree node and tree acceptance ([P1], GPU-Resident
 * Speculation Loop: the acceptance kernel walks the tree from the root and
 * follows the child whose token equals the greedy prediction of its parent;
 * the step commits the accepted draft nodes and the prediction after the
 * last of them). Reads ctrl->n_nodes and ctrl->done when it runs.
 *   logits  fp32 [n_max][V]  rows >= n_nodes are not read.
 *   parent  int32 [n_max]    parent[0] = -1, 0 <= parent[i] < i. A node whose
 *                            parent breaks this is treated as rejected.
 *   token   int32 [n_max]    token of each node (token[0] is the root).
 *   argmax  int32 [n_max]    out: lowest index of each row's maximum.
 *   path    int32 [n_max]    out: path[0..m] = accepted chain from node 0.
 *   ctrl    in/out, see specv_ctrl. When done is set on entry the call only
 *           writes accept_len = 0. Otherwise, with w the deepest accepted
 *           node (lowest index among equally deep ones) and m its depth:
 *           accept_len = m, committed_len += m + 1, root_token = argmax[w],
 *           step += 1, ring_head += m + 1, and done = 1 when
 *           committed_len + n_nodes > ctx_len.
 *   stats   nullable: one record written for the step.
 *   ring    nullable int32 [ring_cap]: the emitted tokens token[path[1..m]]
 *           then argmax[w] go to ring[(ring_head + i) % ring_cap].
 *   workspace  device buffer of tree_argmax_accept_workspace(V, n_max) bytes,
 *           4-byte aligned; its contents need no initialisation.
 * n_max in [1, 16], V in [1, 2^31 - 1]. Alignment: logits 16 bytes.
 */
size_t tree_argmax_accept_workspace(int64_t V, int32_t n_max);
int tree_argmax_accept(const float* logits, int64_t V, int32_t n_max,
                       const int32_t* parent, const int32_t* token,
                       int32_t* argmax, int32_t* path, specv_ctrl* ctrl,
                       specv_step_stats* stats, int32_t* ring, int32_t ring_cap,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tree acceptance from the greedy prediction of each node (for example from
 * w4a8_linear_argmax_T): the same acceptance, commit, ring and statistics as
 * tree_argmax_accept, reading argmax int32 [n_max] instead of logits.
 * n_max in [1, 16].
 */
int tree_accept(const int32_t* argmax, int32_t n_max, const int32_t* parent, const int32_t* token,
                int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* ring,
                int32_t ring_cap, void* stream);

/*
 * The lm_head of a verification step with its argmax epilogue, then tree
 * acceptance from the workgroups' (value, row) pairs ([P1], GPU-Resident
 * Speculation Loop: the greedy prediction of each node and the acceptance
 * run on the device after the forward pass). The same results as
 * w4a8_linear_argmax_T (y not written) followed by tree_accept, in two
 * launches instead of three: the acceptance kernel finishes each node's
 * argmax itself.
 *   wq, ws, xq, xs  the lm_head and the final rows of the T = n_max nodes,
 *                   as w4a8_linear_argmax_T.
 *   argmax   nullable int32 [T] out: each node's greedy prediction.
 *   parent, token, path, ctrl, stats, ring, ring_cap  as tree_argmax_accept.
 *   workspace  w4a8_linear_argmax_workspace(T, N, K) bytes, 8-byte aligned,
 *              no initialisation needed.
 * T in [1, 16]; other shapes, ranges and alignments as w4a8_linear_argmax_T.
 */
int w4a8_linear_argmax_accept_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                                int32_t T, int32_t N, int32_t K, const int32_t* parent,
                                const int32_t* token, int32_t* argmax, int32_t* path, specv_ctrl* ctrl,
                                specv_step_stats* stats, int32_t* ring, int32_t ring_cap, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * KV-cache compaction of the accepted path ([P1], GPU-Resident Speculation
 * Loop: a compaction kernel moves the keys and values of the accepted path
 * into place; [P3], KV transaction model: rows past the committed pointer
 * are dead). Tree node i of the step was written at row L + i. Reads
 * m = ctrl->accept_len and L = ctrl->committed_len - m - 1 when it runs, i.e.
 * it runs after tree_argmax_accept of the same step, and moves row
 * L + path[j] to row L + j for j = 1..m in every layer and KV head, with the
 * result of doing so in increasing j. m == 0 moves nothing.
 *   k_cache, v_cache  fp16 bits [n_layers][n_kv_heads][capacity][head_dim]
 *   path              int32 [m+1] from tree_argmax_accept
 * head_dim a multiple of 8 in [8, 512]; n_layers, n_kv_heads >= 1;
 * capacity >= 1. Alignment: caches 16 bytes.
 */
int kv_compact(uint16_t* k_cache, uint16_t* v_cache, int32_t n_layers, int32_t n_kv_heads,
               int32_t capacity, int32_t head_dim, const int32_t* path,
               const specv_ctrl* ctrl, void* stream);


/*
 * A Qwen2.5-shaped decoder in the W4A8 format, for the tree-masked forward
 * of a verification step ([P1], GPU-Resident Speculation Loop: each step runs
 * the forward pass over the tree, in which each node attends to the
 * committed cache and to its ancestors; Small-Batch Verification Kernels:
 * chunked attention with a merge pass, query heads sharing a KV head read
 * each key and value once). The last holds for groups of at most 8 query
 * heads with n_heads*head_dim <= 1024 and at most 32 chunks of 256 cache
 * rows; other shapes run one attention workgroup per query head, whose
 * repeated reads of a group's rows are served by the L2 cache. Results are
 * the same bits either way. Host struct of device pointers; per-layer
 * tensors are stacked along a leading layer axis. With
 * QKV = (n_heads + 2*n_kv_heads)*head_dim, A = n_heads*head_dim,
 * H = hidden, I = inter, V = vocab. Every matrix is in the packed tile
 * layout of w4a8_pack_weights; a layer's matrix starts
 * w4a8_packed_weight_bytes(rows, K) bytes (and w4a8_packed_scale_bytes
 * bytes for its scales) after the previous layer's:
 *   w_qkv, s_qkv    [layers] x packed (QKV rows, K = H): q rows, then k
 *                   rows, then v rows
 *   w_o, s_o        [layers] x packed (H rows, K = A)
 *   w_gu, s_gu      [layers] x packed (2I rows, K = H): gate and up rows
 *                   alternating in blocks of 8 (gate rows 8b..8b+7, then up
 *                   rows 8b..8b+7, for b = 0 .. I/8 - 1), so that each
 *                   16-row tile of the linear holds gate row i and up row i
 *                   and its epilogue writes silu(gate) * up
 *   w_down, s_down  [layers] x packed (H rows, K = I)
 *   norm_attn, norm_mlp  fp32 [layers][H]; norm_final fp32 [H]
 *   w_lm, s_lm      packed (V rows, K = H); the embedding of a token is its
 *                   dequantised lm_head row (tied weights)
 *   rope_cos, rope_sin  fp32 [max_pos][head_dim/2] (specv_rope_table)
 *   k_cache, v_cache    fp16 bits [layers][n_kv_heads][kv_capacity][head_dim]
 * A step with committed length L and n nodes writes the K/V rows of node i
 * at row L + i and gives node i the logical position L + depth(i). Scores
 * are scaled by 1/sqrt(head_dim); attention runs in chunks of 256 logical
 * positions merged in a second pass; every sum uses the fixed 16-slot order;
 * exp is a fixed Cody-Waite plus degree-7 polynomial evaluation, so results
 * are bit-reproducible. Limits: n_heads/n_kv_heads <= 16; head_dim a
 * multiple of 16 in [16, 128]; hidden, inter and n_heads*head_dim multiples
 * of 32; hidden, inter <= 16384; n_heads*head_dim <= 8192;
 * max_pos >= kv_capacity (a rotary row for every position a step reaches);
 * 4*n_heads*(ceil(kv_capacity/256)+1) <= 64 KiB. The norm weights are
 * 16-byte aligned.
 */
typedef struct {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab, max_pos;
    float eps;          /* RMSNorm epsilon */
    int32_t kv_capacity;
    const uint8_t* w_qkv;  const uint16_t* s_qkv;
    const uint8_t* w_o;    const uint16_t* s_o;
    const uint8_t* w_gu;   const uint16_t* s_gu;
    const uint8_t* w_down; const uint16_t* s_down;
    const float* norm_attn; const float* norm_mlp; const float* norm_final;
    const uint8_t* w_lm;   const uint16_t* s_lm;
    const float* rope_cos; const float* rope_sin;
    uint16_t* k_cache; uint16_t* v_cache;
} specv_model;

/* Rotary table (host memory): for position p < max_pos and pair i < hd/2,
 * the angle p * theta^(-2i/hd) evaluated in double, cos and sin rounded to
 * fp32. Copy the tables to the device for specv_model. */
int specv_rope_table(float* cos_host, float* sin_host, int32_t max_pos, int32_t head_dim, double theta);

/* Workspace bytes of one step with up to n_max nodes (0 on bad arguments). */
size_t spec_step_workspace(const specv_model* m, int32_t n_max);

/*
 * One verification step: the tree-masked forward over ctrl->n_nodes nodes
 * (parent/token as in tree_argmax_accept), then tree_argmax_accept and
 * kv_compact, with the same control-state semantics.
 *   logits  nullable fp32 [n_max][V] out (16-byte aligned): every node's
 *           logits. When NULL they are not written: the lm_head reduces its
 *           rows to each node's (maximum, lowest index) in its epilogue, and
 *           acceptance reads those ([P3]'s greedy rule needs no more).
 *   argmax, path int32 [n_max].
 *   workspace  spec_step_workspace(m, n_max) bytes, 256-byte aligned,
 *              zero-filled before its first use (as for w4a8_linear_T).
 * n_max in [1, 16].
 */
int spec_tree_step(const specv_model* m, specv_ctrl* ctrl, const int32_t* parent,
                   const int32_t* token, int32_t n_max, float* logits, int32_t* argmax,
                   int32_t* path, specv_step_stats* stats, int32_t* ring, int32_t ring_cap,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synthetic drafter of the speculation window (stand-in for the drafter of
 * [P1], Context-Mixing Drafter, which proposes candidates of up to 8 tokens).
 * With L = ctrl->committed_len, d = draws[ctrl->step % draw_rows] (16 words)
 * and D = min(width - 1, 8), the tree of a step is: node 0 the root
 * (ctrl->root_token); nodes 1..D a chain, node k with parent k-1 and token
 * reference[L + k] when d[k] < accept_threshold, else
 * (reference[L + k] + 1 + d[k] % (V - 1)) % V, and d[k] % V once
 * L + k >= reference_len; nodes e in (D, width) get parent (e - D - 1) % D
 * and token d[e] % V. The best-match statistic of the step is D.
 *   reference  int32 [reference_len] device; draws uint32 [draw_rows][16]
 *              device. Both are read while the window runs.
 * 32 bytes; `reserved` is ignored.
 */
typedef struct {
    const int32_t* reference;
    int32_t reference_len;
    int32_t draw_rows;
    const uint32_t* draws;
    uint32_t accept_threshold;
    int32_t reserved;
} specv_drafter;

/* Workspace bytes of a window of the given width (as spec_step_workspace). */
size_t spec_window_workspace(const specv_model* m, int32_t width);

/*
 * Device-resident speculation window ([P1], GPU-Resident Speculation Loop:
 * draft, tree verification, acceptance and compaction run for W steps with
 * no host synchronisation; the host reads the control block and per-step
 * statistics once per window). Each of the W steps drafts a tree of `width`
 * nodes (sets ctrl->n_nodes = width), then runs spec_tree_step's forward,
 * acceptance and compaction. A step that finds done set does nothing but
 * write accept_len = 0 and the record {-1, 0, n_nodes}.
 *   ctrl       device control block (n_nodes is overwritten per step).
 *   stats      specv_step_stats [W] device: record s for step s of the window.
 *   ring       nullable int32 [ring_cap]: the emitted tokens, as in
 *              tree_argmax_accept.
 *   d          drafter; may be NULL only when width == 1 (root-only steps).
 *   width      nodes per step, in [1, 16]; W in [0, 4096], 0 enqueues nothing.
 *   workspace  spec_window_workspace(m, width) bytes, 256-byte aligned,
 *              zero-filled before its first use; it holds the step's tree
 *              and logits, and the window's step counter.
 *   host_readback  nullable host buffer of 32 + 12*W bytes, best pinned
 *              (hipHostMalloc): after the window, ctrl then stats[0..W) are
 *              copied there on `stream`; synchronise before reading.
 * One step's launches are captured once into a HIP graph (on a stream the
 * library creates) and replayed W times on `stream`; the executable graph is
 * kept for the process, keyed by every argument except W and
 * host_readback. At most 32 are kept: the least recently used one is then
 * retired, and destroyed only after its last enqueued window has finished
 * (an event recorded after that window's replays), so windows still queued
 * on any stream are never cut short. Calls from several threads are
 * serialised from the graph lookup to the last replay's enqueue.
 * Windows that share a workspace, control block or cache must not overlap.
 */
int spec_window_run(const specv_model* m, specv_ctrl* ctrl, specv_step_stats* stats,
                    int32_t* ring, int32_t ring_cap, const specv_drafter* d, int32_t width,
                    int32_t W, void* workspace, size_t workspace_bytes, void* host_readback,
                    void* stream);

/*
 * Context-mixing drafter ([P1], Draft-Free Drafting From Web Context: every
 * position of the token history computes the length of its match with the
 * current suffix, at orders up to 8; the best positions' continuations are
 * blended into a weighted trie, weighted by a fixed function of the match
 * length; the most probable prefix-closed node set is the next tree).
 * The stream s[0..n) is the committed tokens followed by the pending root
 * s[n-1]. Position p <= n-2 matches with length l(p), the largest
 * l <= min(max_order, p + 1) with s[p-i] == s[n-1-i] for i < l. The
 * candidates are the `candidates` positions with l >= 1 largest by (l, p);
 * candidate p continues with s[p+1 .. min(p + depth, n - 1)]. A trie node is
 * a prefix of some continuation, weighing the sum of weight[l(p)] over the
 * candidates that continue with it. The tree keeps the width - 1 nodes
 * largest by (weight, smaller depth, earlier first candidate), which is
 * prefix-closed; node 0 is the root (parent -1), then the kept nodes by
 * depth and rank. The step's best match is the first candidate's l (0 if
 * none). Everything is integer, so results are exact.
 * 48 bytes.
 */
typedef struct {
    int32_t max_order;   /* match orders up to this, in [1, 8] */
    int32_t candidates;  /* positions kept, in [1, 32] */
    int32_t depth;       /* continuation tokens per candidate, in [1, 8] */
    uint32_t weight[9];  /* weight[l], l = 1..8, in [1, 2^24]; weight[0] ignored */
} specv_cm_params;

/* Workspace bytes of cm_draft for a stream of n tokens (0 if invalid). */
size_t cm_draft_workspace(int32_t n, const specv_cm_params* p);

/*
 * One tree from a token stream ([P1], Draft-Free Drafting From Web Context).
 *   stream      int32 [n] device, n >= 1: committed tokens, then the root.
 *   p           host parameters, validated as documented above.
 *   width       tree size limit, in [1, 16].
 *   parent, token  int32 [width] device: the tree's first nodes.
 *   out         int32 [2] device: node count (1..width), best match length.
 *   workspace   cm_draft_workspace(n, p) bytes, 4-byte aligned (any content).
 * Returns SPECV_E_SHAPE, SPECV_E_INVAL, SPECV_E_ALIGN or SPECV_E_WORKSPACE
 * without enqueueing anything on bad arguments.
 */
int cm_draft(const int32_t* stream, int32_t n, const specv_cm_params* p, int32_t width, int32_t* parent,
             int32_t* token, int32_t* out, void* workspace, size_t workspace_bytes, void* stream_handle);

/* Workspace bytes of a context-mixing window (0 if invalid). */
size_t spec_window_cm_workspace(const specv_model* m, int32_t width, int32_t ring_cap, const specv_cm_params* p);

/*
 * Speculation window drafted by the context-mixing drafter: as
 * spec_window_run, with each step's tree drafted from the token history by
 * the drafter above (ctrl->n_nodes becomes the tree's size, at most width;
 * the step's best_match record is the drafter's). The history is the ring:
 * ring[i] holds the token at position i of the stream, so the caller fills
 * ring[0..L] with the committed tokens and the root (L = committed_len) and
 * sets ring_head = L + 1; ring_cap must exceed the context limit so the
 * ring never wraps. A step whose ring does not hold the stream (ring_head !=
 * committed_len + 1, or ring[committed_len] != root_token) drafts the root
 * alone.
 *   ring       int32 [ring_cap] device, required.
 *   p          host drafter parameters.
 *   workspace  spec_window_cm_workspace(m, width, ring_cap, p) bytes,
 *              256-byte aligned, zero-filled before its first use.
 * Other arguments, the graph cache and the readback are as in
 * spec_window_run.
 */
int spec_window_run_cm(const specv_model* m, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* ring,
                       int32_t ring_cap, const specv_cm_params* p, int32_t width, int32_t W, void* workspace,
                       size_t workspace_bytes, void* host_readback, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPECV_H */
