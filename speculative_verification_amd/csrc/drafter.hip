// Context-mixing drafter (GPU-Resident Speculative Decoding for In-Browser
// LLM Inference with WebGPU, Draft-Free Drafting From Web Context): every
// position of the token stream computes the length of its match with the
// current suffix, a selection by rank keeps the best positions of each
// workgroup, and one workgroup merges the continuations of the overall best
// into a weighted trie and emits its most probable prefix-closed node set as
// the next tree. Weights are a fixed integer function of the match length,
// so the result is exact.
//
// The stream s[0..n) is the committed tokens followed by the pending root
// s[n-1]. Position p in [0, n-2] matches with length l(p), the largest
// l <= min(max_order, p + 1) with s[p - i] == s[n - 1 - i] for i < l. The
// candidates are the `candidates` positions with l >= 1 that are largest by
// (l, p). Candidate k continues with c_k = s[p+1 .. min(p + depth, n - 1)].
// A trie node is a prefix P of some continuation; its weight is the sum of
// weight[l] over the candidates whose continuation starts with P, and its
// creation order is (first candidate with that prefix, depth). The tree keeps
// the width - 1 nodes largest by (weight, smaller depth, earlier creation):
// a prefix-closed set, since no child outweighs its parent. Node 0 is the
// root; the kept nodes follow by depth, then by rank.
#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kScanThreads = 256;
constexpr int kMergeChunk = 1024;  // keys merged per round in the tree kernel

// Candidate key: match length in bits 24..27, position below (keys of
// positions without a match are 0, which sort last).
__device__ __forceinline__ uint32_t cm_key(int l, int p) { return l > 0 ? ((uint32_t)l << 24) | (uint32_t)p : 0u; }

// Stream length and history, from the control block when the drafter runs
// inside a window (the ring holds the stream: position i at ring[i]), or as
// given. Returns 0 when the history cannot be used (done, or a ring that
// does not hold the whole stream), so only the root is drafted.
__device__ __forceinline__ int cm_stream_len(const specv_ctrl* ctrl, int n_given, int cap,
                                             const int32_t* __restrict__ s) {
    if (!ctrl) return n_given;
    if (ctrl->done) return 0;
    const int n = ctrl->committed_len + 1;
    if (ctrl->ring_head != n || n > cap || s[n - 1] != ctrl->root_token) return 0;
    return n;
}

// Match lengths of 256 positions and the workgroup's best `cands` keys.
// Each thread loads its position's last 8 tokens and the suffix's at once
// (one memory round trip), then counts the matching run. The best keys go
// to their ranks, as in the tree kernel's merge (nonzero keys are
// distinct); places no key takes hold zero.
__global__ __launch_bounds__(kScanThreads) void cm_scan_kernel(const int32_t* __restrict__ s, int n_given, int cap,
                                                               const specv_ctrl* __restrict__ ctrl, int max_order,
                                                               int cands, uint32_t* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint32_t key[kScanThreads];
    __shared__ uint32_t best[32];
    const int n = cm_stream_len(ctrl, n_given, cap, s);
    const int p = blockIdx.x * kScanThreads + threadIdx.x;
    int l = 0;
    if (p + 1 < n) {
        int cur[8], suf[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const bool in = i < max_order && i <= p;
            cur[i] = in ? s[p - i] : 0;
            suf[i] = in ? s[n - 1 - i] : 0;
        }
        bool run = true;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            run = run && i < max_order && i <= p && cur[i] == suf[i];
            l += run;
        }
    }
    const uint32_t x = cm_key(l, p);
    key[threadIdx.x] = x;
    if (threadIdx.x < 32) best[threadIdx.x] = 0u;
    __syncthreads();
    if (x != 0u) {
        int rank = 0;
        const uint4* key4 = reinterpret_cast<const uint4*>(key);
        for (int j = 0; j < kScanThreads / 4; j++) {  // every lane reads the same words
            const uint4 v = key4[j];
            rank += (v.x > x) + (v.y > x) + (v.z > x) + (v.w > x);
        }
        if (rank < cands) best[rank] = x;
    }
    __syncthreads();
    if (threadIdx.x < cands) part[blockIdx.x * cands + threadIdx.x] = best[threadIdx.x];
}

// One workgroup: global best candidates, trie weights, selection and output.
// At most 32 candidates of depth at most 8: thread (k, d) = (tid / 8, tid % 8)
// stands for the prefix of length d + 1 of candidate k.
__global__ __launch_bounds__(256) void cm_tree_kernel(const int32_t* __restrict__ s, int n_given, int cap,
                                                      specv_ctrl* __restrict__ ctrl, const uint32_t* __restrict__ part,
                                                      int nparts, const specv_cm_params prm, int width,
                                                      int32_t* __restrict__ parent, int32_t* __restrict__ token,
                                                      int32_t* __restrict__ n_nodes_out,
                                                      int32_t* __restrict__ best_match_out,
                                                      specv_step_stats* __restrict__ stats,
                                                      const int32_t* __restrict__ wcounter) {
    __shared__ __attribute__((aligned(16))) uint32_t pool[kMergeChunk + 32 + 4];
    __shared__ uint32_t keys[32];
    __shared__ __attribute__((aligned(16))) int32_t cont[32][8];
    __shared__ int clen[32];
    __shared__ uint32_t cw[32];
    __shared__ __attribute__((aligned(16))) uint32_t wt[32][8];
    __shared__ __attribute__((aligned(16))) int rankv[32][8];
    __shared__ int outi[32][8];
    __shared__ int wcount[4];
    const int tid = threadIdx.x;
    const int cands = prm.candidates, depth = prm.depth;
    const int n = cm_stream_len(ctrl, n_given, cap, s);

    // running best `cands` keys over the parts that hold stream positions
    // (later parts hold only the zero keys of positions without a match),
    // a chunk of parts at a time: the chunk's keys and the best so far form
    // a pool, and each nonzero key goes to its rank, the number of pool keys
    // above it (nonzero keys are distinct, their positions differ), if that
    // is below `cands`; the places no key takes stay zero. This is the
    // descending order's first `cands` keys, as a sort of the pool gives.
    const int used = min(nparts, (n + kScanThreads - 1) / kScanThreads);
    const int total = used * cands;
    if (tid < 32) keys[tid] = 0u;
    for (int base = 0; base < total; base += kMergeChunk) {
        const int m = min(kMergeChunk, total - base);
        const int np = m + cands, np4 = (np + 3) >> 2;
        __syncthreads();  // the previous round's keys are written
        for (int i = tid; i < 4 * np4; i += 256) pool[i] = i < m ? part[base + i] : i < np ? keys[i - m] : 0u;
        __syncthreads();
        if (tid < 32) keys[tid] = 0u;
        __syncthreads();
        const uint4* pool4 = reinterpret_cast<const uint4*>(pool);
        for (int i = tid; i < np; i += 256) {
            const uint32_t x = pool[i];
            if (x == 0u) continue;
            int rank = 0;
            for (int j = 0; j < np4; j++) {  // every lane reads the same words
                const uint4 v = pool4[j];
                rank += (v.x > x) + (v.y > x) + (v.z > x) + (v.w > x);
            }
            if (rank < cands) keys[rank] = x;
        }
    }
    __syncthreads();
    // candidates and their continuations
    if (tid < 32) {
        const uint32_t kk = tid < cands ? keys[tid] : 0u;
        const int l = (int)(kk >> 24), p = (int)(kk & 0xFFFFFFu);
        const int len = kk ? min(depth, n - 1 - p) : 0;
        clen[tid] = len;
        cw[tid] = kk ? prm.weight[l] : 0u;
        for (int d = 0; d < 8; d++) cont[tid][d] = d < len ? s[p + 1 + d] : -1;
    }
    __syncthreads();

    const int k = tid >> 3, d = tid & 7;
    const bool valid = d < clen[k];
    // representative: the first candidate with the same prefix; weight: the
    // sum over every candidate with the same prefix; the parent's
    // representative: the first candidate with the prefix shortened by one.
    // Candidate j has the prefix of length e + 1 when it is longer than e
    // and its continuation differs from this one at no depth up to e (a bit
    // mask of the differing depths, from two 16-byte reads of its row).
    int rep = k, prep = k;
    uint32_t w = 0;
    if (valid) {
        const int4 ka = *reinterpret_cast<const int4*>(&cont[k][0]);
        const int4 kb = *reinterpret_cast<const int4*>(&cont[k][4]);
        const uint32_t upto = (2u << d) - 1u, upto1 = (1u << d) - 1u;
        for (int j = 31; j >= 0; j--) {
            const int4 a = *reinterpret_cast<const int4*>(&cont[j][0]);
            const int4 b = *reinterpret_cast<const int4*>(&cont[j][4]);
            const uint32_t diff = (uint32_t)(a.x != ka.x) | (uint32_t)(a.y != ka.y) << 1 |
                                  (uint32_t)(a.z != ka.z) << 2 | (uint32_t)(a.w != ka.w) << 3 |
                                  (uint32_t)(b.x != kb.x) << 4 | (uint32_t)(b.y != kb.y) << 5 |
                                  (uint32_t)(b.z != kb.z) << 6 | (uint32_t)(b.w != kb.w) << 7;
            const int lj = clen[j];
            if (lj > d && (diff & upto) == 0u) {
                w += cw[j];
                rep = j;  // ends at the smallest such j
            }
            if (lj > d - 1 && (diff & upto1) == 0u) prep = j;
        }
    }
    const bool is_node = valid && rep == k;
    wt[k][d] = is_node ? w : 0u;
    __syncthreads();
    // rank among the nodes, reading the weight table 16 bytes at a time
    // (every node weighs at least 1, so a zero entry is not a node)
    int rank = 1 << 20;
    if (is_node) {
        rank = 0;
#pragma unroll 4
        for (int j = 0; j < 32; j++) {
            const uint4 a = *reinterpret_cast<const uint4*>(&wt[j][0]);
            const uint4 b = *reinterpret_cast<const uint4*>(&wt[j][4]);
            const uint32_t row[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t w2 = row[e];
                rank += w2 != 0u && (w2 > w || (w2 == w && (e < d || (e == d && j < k))));
            }
        }
    }
    const bool keep = is_node && rank < width - 1;
    rankv[k][d] = keep ? rank : -1;
    __syncthreads();
    // output position: by depth, then rank
    if (keep) {
        int pos = 1;
#pragma unroll 4
        for (int j = 0; j < 32; j++) {
            const int4 a = *reinterpret_cast<const int4*>(&rankv[j][0]);
            const int4 b = *reinterpret_cast<const int4*>(&rankv[j][4]);
            const int row[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 8; e++) pos += row[e] >= 0 && (e < d || (e == d && row[e] < rank));
        }
        outi[k][d] = pos;
    }
    // the number of kept nodes: one per thread, summed over the workgroup
    {
        const unsigned long long b = __ballot(keep);
        if ((tid & 63) == 0) wcount[tid >> 6] = __popcll(b);
    }
    __syncthreads();
    if (keep) {
        // the parent node is the representative of this prefix shortened by one
        const int par = d > 0 ? outi[prep][d - 1] : 0;
        const int pos = outi[k][d];
        parent[pos] = par;
        token[pos] = cont[k][d];
    }
    if (tid == 0) {
        const int nodes = n > 0 ? 1 + wcount[0] + wcount[1] + wcount[2] + wcount[3] : 1;
        const int bm = (n > 0 && keys[0]) ? (int)(keys[0] >> 24) : 0;
        parent[0] = -1;
        if (ctrl) {
            if (!ctrl->done) {
                token[0] = ctrl->root_token;
                ctrl->n_nodes = nodes;
            }
            if (stats) stats[*wcounter].best_match = ctrl->done ? 0 : bm;
        } else {
            token[0] = n > 0 ? s[n - 1] : 0;
            *n_nodes_out = nodes;
            *best_match_out = bm;
        }
    }
}

static int cm_scan_parts(int cap) { return (cap + kScanThreads - 1) / kScanThreads; }

bool cm_params_ok(const specv_cm_params* p) {
    if (!p || p->max_order < 1 || p->max_order > 8 || p->candidates < 1 || p->candidates > 32 || p->depth < 1 ||
        p->depth > 8)
        return false;
    for (int l = 1; l <= 8; l++)
        if (p->weight[l] < 1 || p->weight[l] > (1u << 24)) return false;
    return true;
}

// Workspace: the per-workgroup keys of the scan.
size_t cm_workspace_bytes(int cap, const specv_cm_params* p) { return (size_t)cm_scan_parts(cap) * p->candidates * 4; }

int enqueue_cm_draft(const int32_t* s, int n_given, int cap, specv_ctrl* ctrl, const specv_cm_params* p, int width,
                     int32_t* parent, int32_t* token, int32_t* n_nodes_out, int32_t* best_match_out,
                     specv_step_stats* stats, const int32_t* wcounter, void* workspace, hipStream_t st) {
    uint32_t* part = static_cast<uint32_t*>(workspace);
    const int parts = cm_scan_parts(cap);
    hipLaunchKernelGGL(cm_scan_kernel, dim3(parts), dim3(kScanThreads), 0, st, s, n_given, cap, ctrl, p->max_order,
                       p->candidates, part);
    hipLaunchKernelGGL(cm_tree_kernel, dim3(1), dim3(256), 0, st, s, n_given, cap, ctrl, part, parts, *p, width,
                       parent, token, n_nodes_out, best_match_out, stats, wcounter);
    return launch_status();
}

}  // namespace specv

extern "C" size_t cm_draft_workspace(int32_t n, const specv_cm_params* p) {
    using namespace specv;
    if (n < 1 || n > (1 << 24) || !cm_params_ok(p)) return 0;
    return cm_workspace_bytes(n, p);
}

extern "C" int cm_draft(const int32_t* stream, int32_t n, const specv_cm_params* p, int32_t width, int32_t* parent,
                        int32_t* token, int32_t* out, void* workspace, size_t workspace_bytes, void* stream_handle) {
    using namespace specv;
    if (n < 1 || n > (1 << 24) || width < 1 || width > 16) return SPECV_E_SHAPE;
    if (!stream || !p || !parent || !token || !out) return SPECV_E_INVAL;
    if (!cm_params_ok(p)) return SPECV_E_INVAL;
    if (!aligned(stream, 4) || !aligned(parent, 4) || !aligned(token, 4) || !aligned(out, 4)) return SPECV_E_ALIGN;
    const size_t need = cm_workspace_bytes(n, p);
    if (!workspace || workspace_bytes < need) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 4)) return SPECV_E_ALIGN;
    return enqueue_cm_draft(stream, n, n, nullptr, p, width, parent, token, out, out + 1, nullptr, nullptr,
                            workspace, (hipStream_t)stream_handle);
}
