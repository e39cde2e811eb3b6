// KV-cache compaction of the accepted path (GPU-Resident Speculative
// Decoding for In-Browser LLM Inference with WebGPU, GPU-Resident
// Speculation Loop; rows past the committed pointer are dead, as in the KV
// transaction model of Exact Speculative And Assisted Decoding For A Tiny
// Draft And Qualified Champion).
//
// Each thread owns one 16-byte column chunk of one (layer, K/V, head) plane
// and moves it for every accepted node. It first loads all m source rows,
// then stores all m destinations. Since path[j] >= j, no source row of a
// later node is a destination of an earlier one, so gathering from the
// state before the call equals moving the rows one by one in increasing j.
// Distinct threads touch distinct bytes, so there is no inter-thread hazard.
#include "common.h"

namespace specv {

constexpr int kCompactThreads = 256;
constexpr int kMaxMoves = 15;  // at most 16 nodes, so at most 15 accepted drafts

__global__ __launch_bounds__(kCompactThreads) void kv_compact_kernel(
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int planes, int capacity, int head_dim,
    const int32_t* __restrict__ path, const specv_ctrl* __restrict__ ctrl) {
    const int m_raw = ctrl->accept_len;
    if (m_raw <= 0) return;
    const int m = m_raw > kMaxMoves ? kMaxMoves : m_raw;
    const int L = ctrl->committed_len - m_raw - 1;
    const int cpr = head_dim / 8;  // 16-byte chunks per row
    const int64_t idx = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x;
    if (idx >= (int64_t)2 * planes * cpr) return;
    const int c = (int)(idx % cpr);
    const int64_t pk = idx / cpr;  // plane index over K planes then V planes
    uint16_t* base = (pk < planes ? kc + pk * (int64_t)capacity * head_dim
                                  : vc + (pk - planes) * (int64_t)capacity * head_dim) + 8 * c;
    v4i buf[kMaxMoves];
    bool ok[kMaxMoves];
#pragma unroll
    for (int j = 1; j <= kMaxMoves; j++) {
        ok[j - 1] = false;
        if (j <= m) {
            const int src = L + path[j];
            ok[j - 1] = L >= 0 && path[j] >= j && src < capacity && L + j < capacity;
            if (ok[j - 1]) buf[j - 1] = *reinterpret_cast<const v4i*>(base + (int64_t)src * head_dim);
        }
    }
#pragma unroll
    for (int j = 1; j <= kMaxMoves; j++)
        if (j <= m && ok[j - 1]) *reinterpret_cast<v4i*>(base + (int64_t)(L + j) * head_dim) = buf[j - 1];
}

}  // namespace specv

extern "C" int kv_compact(uint16_t* k_cache, uint16_t* v_cache, int32_t n_layers, int32_t n_kv_heads,
                          int32_t capacity, int32_t head_dim, const int32_t* path,
                          const specv_ctrl* ctrl, void* stream) {
    using namespace specv;
    if (n_layers < 1 || n_kv_heads < 1 || capacity < 1 || head_dim < 8 || head_dim > 512 ||
        head_dim % 8)
        return SPECV_E_SHAPE;
    if ((int64_t)n_layers * n_kv_heads > (1 << 20)) return SPECV_E_SHAPE;
    if (!k_cache || !v_cache || !path || !ctrl) return SPECV_E_INVAL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(path, 4) || !aligned(ctrl, 4))
        return SPECV_E_ALIGN;
    const int planes = n_layers * n_kv_heads;
    const int64_t threads = (int64_t)2 * planes * (head_dim / 8);
    const int blocks = (int)((threads + kCompactThreads - 1) / kCompactThreads);
    hipLaunchKernelGGL(kv_compact_kernel, dim3(blocks), dim3(kCompactThreads), 0, (hipStream_t)stream,
                       k_cache, v_cache, planes, capacity, head_dim, path, ctrl);
    return launch_status();
}
