// Greedy argmax per tree node and tree acceptance, driven by device-resident
// control state (GPU-Resident Speculative Decoding for In-Browser LLM
// Inference with WebGPU, GPU-Resident Speculation Loop).
//
// Two launches, both reading ctrl at run time:
//  1. argmax_partial_kernel: grid (chunks, n_max). Each workgroup reduces
//     4096 logits of one node to (max, lowest index). The combine rule
//     "larger value, or equal value and lower index" is a total order on
//     (value, -index) with -0 == +0, so any reduction shape gives the same
//     winner: the lowest index of the row maximum.
//  2. accept_kernel: one workgroup. Finishes each node's argmax from the
//     partials, then one thread walks the tree: node i is accepted when its
//     parent is accepted and token[i] equals the parent's prediction; the
//     deepest accepted node (lowest index among equals) ends the path. It
//     commits the step in ctrl, appends the emitted tokens to the ring and
//     writes the step statistics.
#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kArgThreads = 256;
constexpr int kArgChunk = 4096;  // logits per partial workgroup
constexpr int kMaxNodes = 16;

__device__ __forceinline__ void wave_best(float& v, int& i, int width) {
    for (int off = width / 2; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off, width);
        const int oi = __shfl_xor(i, off, width);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

__global__ __launch_bounds__(kArgThreads) void argmax_partial_kernel(
    const float* __restrict__ logits, int64_t V, const specv_ctrl* __restrict__ ctrl,
    Best* __restrict__ part, int chunks) {
    const int node = blockIdx.y;
    if (ctrl->done || node >= ctrl->n_nodes) return;
    const int64_t start = (int64_t)blockIdx.x * kArgChunk;
    const int64_t end = start + kArgChunk < V ? start + kArgChunk : V;
    const float* row = logits + (int64_t)node * V;

    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    for (int64_t k = start + threadIdx.x; k < end; k += kArgThreads) {
        const float v = row[k];
        if (better(v, (int)k, bv, bi)) {
            bv = v;
            bi = (int)k;
        }
    }
    wave_best(bv, bi, 64);
    __shared__ Best wb[kArgThreads / 64];
    if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = Best{bv, bi};
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgThreads / 64; w++)
            if (better(wb[w].v, wb[w].i, bv, bi)) {
                bv = wb[w].v;
                bi = wb[w].i;
            }
        part[(int64_t)node * chunks + blockIdx.x] = Best{bv, bi};
    }
}

__global__ __launch_bounds__(kArgThreads) void accept_kernel(
    const Best* __restrict__ part, int chunks, const int32_t* __restrict__ amax_in, int n_max,
    const int32_t* __restrict__ parent,
    const int32_t* __restrict__ token, int32_t* __restrict__ argmax_out, int32_t* __restrict__ path,
    specv_ctrl* __restrict__ ctrl, specv_step_stats* __restrict__ stats_base, int32_t* __restrict__ wcounter,
    int32_t* __restrict__ ring, int ring_cap) {
    __shared__ int s_amax[kMaxNodes];
    __shared__ int s_acc[kMaxNodes];
    __shared__ int s_depth[kMaxNodes];
    const int done = ctrl->done;
    int n = ctrl->n_nodes;
    n = n < 1 ? 1 : (n > n_max ? n_max : n);
    // Statistics of a window step go to the record its counter names.
    specv_step_stats* stats = stats_base ? stats_base + (wcounter ? *wcounter : 0) : nullptr;
    __syncthreads();
    if (done) {
        if (threadIdx.x == 0) {
            ctrl->accept_len = 0;
            if (stats) {
                stats->accepted = -1;
                stats->width = n;
            }
            if (wcounter) *wcounter = *wcounter + 1;
        }
        return;
    }
    // The tree goes to LDS while the argmax partials are read.
    __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes];
    __shared__ Best s_grp[kArgThreads / 16];
    if (threadIdx.x < n) {
        s_par[threadIdx.x] = parent[threadIdx.x];
        s_tok[threadIdx.x] = token[threadIdx.x];
    }
    if (amax_in) {
        if (threadIdx.x < n) s_amax[threadIdx.x] = amax_in[threadIdx.x];
    } else {
        // tpn = 256 / (n rounded up to a power of two) threads per node, each
        // taking every tpn-th partial, four loads in flight; the best of each
        // 16-lane group, then of the node's groups (order-free).
        int np = 1;
        while (np < n) np <<= 1;
        const int tpn = kArgThreads / np;
        const int node = threadIdx.x / tpn, sub = threadIdx.x - node * tpn;
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        if (node < n) {
            const Best* pn = part + (int64_t)node * chunks;
            int c = sub;
            for (; c + 3 * tpn < chunks; c += 4 * tpn) {
                const Best b0 = pn[c], b1 = pn[c + tpn], b2 = pn[c + 2 * tpn], b3 = pn[c + 3 * tpn];
                if (better(b0.v, b0.i, bv, bi)) { bv = b0.v; bi = b0.i; }
                if (better(b1.v, b1.i, bv, bi)) { bv = b1.v; bi = b1.i; }
                if (better(b2.v, b2.i, bv, bi)) { bv = b2.v; bi = b2.i; }
                if (better(b3.v, b3.i, bv, bi)) { bv = b3.v; bi = b3.i; }
            }
            for (; c < chunks; c += tpn) {
                const Best b = pn[c];
                if (better(b.v, b.i, bv, bi)) {
                    bv = b.v;
                    bi = b.i;
                }
            }
        }
        best16(bv, bi);
        if ((threadIdx.x & 15) == 0) s_grp[threadIdx.x >> 4] = Best{bv, bi};
        __syncthreads();
        if (threadIdx.x < n) {
            const int g0 = threadIdx.x * (tpn / 16), ng = tpn / 16;
            Best b = s_grp[g0];
            for (int k = 1; k < ng; k++)
                if (better(s_grp[g0 + k].v, s_grp[g0 + k].i, b.v, b.i)) b = s_grp[g0 + k];
            s_amax[threadIdx.x] = b.i;
            if (argmax_out) argmax_out[threadIdx.x] = b.i;
        }
    }
    __syncthreads();
    if (threadIdx.x != 0) return;

    s_acc[0] = 1;
    s_depth[0] = 0;
    for (int i = 1; i < n; i++) {
        const int p = s_par[i];
        if (p < 0 || p >= i) {
            s_acc[i] = 0;
            s_depth[i] = 0;
        } else {
            s_acc[i] = s_acc[p] && s_tok[i] == s_amax[p];
            s_depth[i] = s_depth[p] + 1;
        }
    }
    int w = 0;
    for (int i = 1; i < n; i++)
        if (s_acc[i] && s_depth[i] > s_depth[w]) w = i;
    const int m = s_depth[w];
    for (int i = w, j = m; j >= 0; j--) {
        s_path[j] = i;
        path[j] = i;
        i = j > 0 ? s_par[i] : i;
    }
    const int bonus = s_amax[w];
    const int head = ctrl->ring_head;
    if (ring && ring_cap > 0)
        for (int j = 0; j <= m; j++) ring[(uint32_t)(head + j) % (uint32_t)ring_cap] = j < m ? s_tok[s_path[j + 1]] : bonus;
    const int L = ctrl->committed_len + m + 1;
    ctrl->accept_len = m;
    ctrl->committed_len = L;
    ctrl->root_token = bonus;
    ctrl->step = ctrl->step + 1;
    ctrl->ring_head = head + m + 1;
    if (L + ctrl->n_nodes > ctrl->ctx_len) ctrl->done = 1;
    if (stats) {
        stats->accepted = m;
        stats->width = n;
    }
    if (wcounter) *wcounter = *wcounter + 1;
}

inline int argmax_chunks(int64_t V) { return (int)((V + kArgChunk - 1) / kArgChunk); }

}  // namespace specv

extern "C" size_t tree_argmax_accept_workspace(int64_t V, int32_t n_max) {
    if (V < 1 || n_max < 1) return 0;
    return (size_t)n_max * (size_t)specv::argmax_chunks(V) * sizeof(specv::Best);
}

namespace specv {

int enqueue_argmax_accept(const float* logits, int64_t V, int n_max, const int32_t* parent,
                          const int32_t* token, int32_t* argmax, int32_t* path, specv_ctrl* ctrl,
                          specv_step_stats* stats, int32_t* wcounter, int32_t* ring, int32_t ring_cap,
                          void* partials, hipStream_t s) {
    const int chunks = argmax_chunks(V);
    Best* part = static_cast<Best*>(partials);
    hipLaunchKernelGGL(argmax_partial_kernel, dim3(chunks, n_max), dim3(kArgThreads), 0, s, logits, V, ctrl,
                       part, chunks);
    const int rc = launch_status();
    if (rc != SPECV_OK) return rc;
    return enqueue_accept(part, chunks, nullptr, n_max, parent, token, argmax, path, ctrl, stats, wcounter, ring,
                          ring_cap, s);
}

int enqueue_accept(const Best* part, int chunks, const int32_t* amax_in, int n_max, const int32_t* parent,
                   const int32_t* token, int32_t* argmax_out, int32_t* path, specv_ctrl* ctrl,
                   specv_step_stats* stats, int32_t* wcounter, int32_t* ring, int32_t ring_cap, hipStream_t s) {
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kArgThreads), 0, s, part, chunks, amax_in, n_max, parent, token,
                       argmax_out, path, ctrl, stats, wcounter, ring, ring_cap);
    return launch_status();
}

}  // namespace specv

extern "C" int tree_argmax_accept(const float* logits, int64_t V, int32_t n_max,
                                  const int32_t* parent, const int32_t* token, int32_t* argmax,
                                  int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats,
                                  int32_t* ring, int32_t ring_cap, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    using namespace specv;
    if (V < 1 || V > 0x7fffffffLL || n_max < 1 || n_max > kMaxNodes) return SPECV_E_SHAPE;
    if (!logits || !parent || !token || !argmax || !path || !ctrl) return SPECV_E_INVAL;
    if (ring && ring_cap < 1) return SPECV_E_INVAL;
    if (!aligned(logits, 16) || !aligned(parent, 4) || !aligned(token, 4) || !aligned(argmax, 4) ||
        !aligned(path, 4) || !aligned(ctrl, 4) || !aligned(stats, 4) || !aligned(ring, 4))
        return SPECV_E_ALIGN;
    const size_t need = tree_argmax_accept_workspace(V, n_max);
    if (!workspace || workspace_bytes < need) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 4)) return SPECV_E_ALIGN;
    return enqueue_argmax_accept(logits, V, n_max, parent, token, argmax, path, ctrl, stats, nullptr, ring,
                                 ring_cap, workspace, (hipStream_t)stream);
}

extern "C" int tree_accept(const int32_t* argmax, int32_t n_max, const int32_t* parent, const int32_t* token,
                           int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* ring,
                           int32_t ring_cap, void* stream) {
    using namespace specv;
    if (n_max < 1 || n_max > kMaxNodes) return SPECV_E_SHAPE;
    if (!argmax || !parent || !token || !path || !ctrl) return SPECV_E_INVAL;
    if (ring && ring_cap < 1) return SPECV_E_INVAL;
    if (!aligned(argmax, 4) || !aligned(parent, 4) || !aligned(token, 4) || !aligned(path, 4) ||
        !aligned(ctrl, 4) || !aligned(stats, 4) || !aligned(ring, 4))
        return SPECV_E_ALIGN;
    return enqueue_accept(nullptr, 0, argmax, n_max, parent, token, nullptr, path, ctrl, stats, nullptr, ring,
                          ring_cap, (hipStream_t)stream);
}

// The lm_head with its argmax epilogue, then acceptance straight from the
// workgroups' (value, row) pairs: two launches, where w4a8_linear_argmax_T
// followed by tree_accept takes three (the finishing pass of the argmax is
// the acceptance kernel's first phase).
extern "C" int w4a8_linear_argmax_accept_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                                           const float* xs, int32_t T, int32_t N, int32_t K,
                                           const int32_t* parent, const int32_t* token, int32_t* argmax,
                                           int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats,
                                           int32_t* ring, int32_t ring_cap, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    using namespace specv;
    if (T < 1 || T > kMaxNodes || N < 1 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32)
        return SPECV_E_SHAPE;
    if (packed_weight_bytes(N, K) >= (int64_t)1 << 31 || !linear_argmax_supported(T, N, K)) return SPECV_E_SHAPE;
    if (!wq || !ws || !xq || !xs || !parent || !token || !path || !ctrl) return SPECV_E_INVAL;
    if (ring && ring_cap < 1) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(ws, 2) || !aligned(xs, 4) || !aligned(parent, 4) ||
        !aligned(token, 4) || !aligned(argmax, 4) || !aligned(path, 4) || !aligned(ctrl, 4) ||
        !aligned(stats, 4) || !aligned(ring, 4))
        return SPECV_E_ALIGN;
    const size_t need = w4a8_linear_argmax_workspace(T, N, K);
    if (!workspace || workspace_bytes < need) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 8)) return SPECV_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    Best* part = static_cast<Best*>(workspace);
    const int rc = linear_enqueue(wq, ws, xq, xs, nullptr, part, T, N, K, nullptr, s);
    if (rc != SPECV_OK) return rc;
    return enqueue_accept(part, linear_argmax_chunks(T, N, K), nullptr, T, parent, token, argmax, path, ctrl, stats,
                          nullptr, ring, ring_cap, s);
}
