// Device-resident speculation window (GPU-Resident Speculative Decoding for
// In-Browser LLM Inference with WebGPU, GPU-Resident Speculation Loop):
// W steps of draft -> tree-masked forward -> acceptance -> compaction run
// back to back with no host decision in between, because every kernel reads
// its dynamic state (committed length, node count, root token, step, done)
// from the device control block. The window ends with one copy of the
// 32-byte control block and 12 bytes of statistics per step to the host.
//
// One step is captured once into a HIP graph (its launches never change;
// only the control block does) and replayed W times on the caller's stream.
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"

namespace specv {

// Synthetic drafter standing in for the context-mixing drafter (the pages'
// drafter extends a candidate by at most 8 tokens): node 0 is the root with
// the last step's bonus token; nodes 1..D (D = min(width-1, 8)) form a chain;
// chain node k copies the reference token at position L+k when its draw is
// below the threshold and otherwise takes a different token; the remaining
// nodes attach round-robin to nodes 0..D-1 with tokens draw mod vocab.
__global__ void draft_kernel(specv_ctrl* ctrl, int width, const int32_t* __restrict__ ref, int ref_len,
                             const uint32_t* __restrict__ draws, int draw_rows, uint32_t threshold, int vocab,
                             int32_t* __restrict__ parent, int32_t* __restrict__ token,
                             specv_step_stats* __restrict__ stats, const int32_t* __restrict__ wcounter) {
    if (threadIdx.x != 0) return;
    if (ctrl->done) {
        if (stats) stats[*wcounter].best_match = 0;
        return;
    }
    const int L = ctrl->committed_len;
    const int D = width - 1 < 8 ? width - 1 : 8;
    const uint32_t* dr = draws + (size_t)((uint32_t)ctrl->step % (uint32_t)draw_rows) * 16;
    parent[0] = -1;
    token[0] = ctrl->root_token;
    for (int k = 1; k <= D; k++) {
        parent[k] = k - 1;
        const uint32_t d = dr[k];
        if (L + k < ref_len) {
            const int32_t r = ref[L + k];
            token[k] = d < threshold ? r
                                     : (int32_t)(((uint32_t)r + 1u + d % (uint32_t)(vocab - 1)) % (uint32_t)vocab);
        } else {
            token[k] = (int32_t)(d % (uint32_t)vocab);
        }
    }
    for (int e = D + 1; e < width; e++) {
        parent[e] = (e - D - 1) % D;
        token[e] = (int32_t)(dr[e] % (uint32_t)vocab);
    }
    ctrl->n_nodes = width;
    if (stats) stats[*wcounter].best_match = D;
}

// Width-1 steps need no draft: the tree is the root alone.
__global__ void root_only_kernel(specv_ctrl* ctrl, int32_t* __restrict__ parent, int32_t* __restrict__ token,
                                 specv_step_stats* __restrict__ stats, const int32_t* __restrict__ wcounter) {
    if (threadIdx.x != 0) return;
    if (ctrl->done) {
        if (stats) stats[*wcounter].best_match = 0;
        return;
    }
    parent[0] = -1;
    token[0] = ctrl->root_token;
    ctrl->n_nodes = 1;
    if (stats) stats[*wcounter].best_match = 0;
}

__global__ void window_begin_kernel(int32_t* wcounter) {
    if (threadIdx.x == 0) *wcounter = 0;
}

enum { kRootOnly = 0, kSynthetic = 1, kContextMixing = 2 };

struct WindowKey {
    specv_model model;
    specv_ctrl* ctrl;
    specv_step_stats* stats;
    int32_t* ring;
    int32_t ring_cap;
    int32_t width;
    int32_t drafter_kind;  // kRootOnly, kSynthetic or kContextMixing
    specv_drafter drafter;
    specv_cm_params cm;
    void* workspace;
    bool operator<(const WindowKey& o) const { return std::memcmp(this, &o, sizeof(WindowKey)) < 0; }
};

// Cached step graphs. An entry keeps its last use (a counter) and an event
// recorded on the caller's stream after the window's last replay. The cache
// holds at most kGraphCacheMax entries; when full, the least recently used
// one is retired: it leaves the map, and its graph is destroyed only once
// its event reports that every replay enqueued so far has finished (checked
// on every later call, without blocking). The lock is held from the lookup
// to the event record, so no thread can retire a graph between another
// thread's lookup and its launches.
constexpr size_t kGraphCacheMax = 32;

struct GraphEntry {
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;  // recorded after the entry's latest window
    uint64_t last_use = 0;
};

struct GraphCache {
    std::mutex mu;
    std::map<WindowKey, GraphEntry> entries;
    std::vector<GraphEntry> retired;  // evicted, waiting for their last window
    uint64_t clock = 0;
    hipStream_t capture_stream = nullptr;
};

static GraphCache& graph_cache() {
    static GraphCache* c = new GraphCache();  // lives for the process
    return *c;
}

static void destroy_entry(GraphEntry& e) {
    if (e.exec) (void)hipGraphExecDestroy(e.exec);
    if (e.done) (void)hipEventDestroy(e.done);
    e.exec = nullptr;
    e.done = nullptr;
}

// Destroys the retired graphs whose windows have all finished. Called with
// the cache lock held.
static void reap_retired(GraphCache& gc) {
    for (size_t i = 0; i < gc.retired.size();) {
        if (hipEventQuery(gc.retired[i].done) == hipSuccess) {
            destroy_entry(gc.retired[i]);
            gc.retired[i] = gc.retired.back();
            gc.retired.pop_back();
        } else {
            (void)hipGetLastError();  // hipErrorNotReady is not an error here
            i++;
        }
    }
}

static int enqueue_window_step(const WindowKey& k, const StepLayout& lay, hipStream_t s) {
    char* ws = static_cast<char*>(k.workspace);
    int32_t* tree = reinterpret_cast<int32_t*>(ws + lay.tree);
    int32_t *parent = tree, *token = tree + 16, *argmax = tree + 32, *path = tree + 48;
    int32_t* wcounter = reinterpret_cast<int32_t*>(ws + lay.wcounter);
    float* logits = nullptr;  // not wanted: acceptance reads the lm_head's argmax pairs
    int rc = SPECV_OK;
    if (k.drafter_kind == kSynthetic) {
        hipLaunchKernelGGL(draft_kernel, dim3(1), dim3(64), 0, s, k.ctrl, k.width, k.drafter.reference,
                           k.drafter.reference_len, k.drafter.draws, k.drafter.draw_rows,
                           k.drafter.accept_threshold, k.model.vocab, parent, token, k.stats, wcounter);
        rc = launch_status();
    } else if (k.drafter_kind == kContextMixing) {
        rc = enqueue_cm_draft(k.ring, 0, k.ring_cap, k.ctrl, &k.cm, k.width, parent, token, nullptr, nullptr, k.stats,
                              wcounter, ws + lay.total, s);
    } else {
        hipLaunchKernelGGL(root_only_kernel, dim3(1), dim3(64), 0, s, k.ctrl, parent, token, k.stats, wcounter);
        rc = launch_status();
    }
    if (rc != SPECV_OK) return rc;
    return enqueue_step(&k.model, k.width, parent, token, logits, argmax, path, k.ctrl, k.stats, wcounter, k.ring,
                        k.ring_cap, ws, lay, s);
}

// The cache entry of a window step, captured into an executable graph on
// first use. Called with the cache lock held.
static int window_graph(GraphCache& gc, const WindowKey& k, const StepLayout& lay, GraphEntry** out) {
    auto it = gc.entries.find(k);
    if (it != gc.entries.end()) {
        *out = &it->second;
        return SPECV_OK;
    }
    if (!gc.capture_stream && hipStreamCreateWithFlags(&gc.capture_stream, hipStreamNonBlocking) != hipSuccess)
        return SPECV_E_HIP;
    // Relaxed capture: kernel attributes set while enqueueing (dynamic LDS
    // limits) are not stream work and may be changed during capture.
    if (hipStreamBeginCapture(gc.capture_stream, hipStreamCaptureModeRelaxed) != hipSuccess) return SPECV_E_HIP;
    const int rc = enqueue_window_step(k, lay, gc.capture_stream);
    hipGraph_t g = nullptr;
    const bool ended = hipStreamEndCapture(gc.capture_stream, &g) == hipSuccess;
    if (rc != SPECV_OK || !ended) {
        if (g) (void)hipGraphDestroy(g);
        (void)hipGetLastError();
        return rc != SPECV_OK ? rc : SPECV_E_HIP;
    }
    GraphEntry e;
    const bool inst = hipGraphInstantiate(&e.exec, g, nullptr, nullptr, 0) == hipSuccess;
    (void)hipGraphDestroy(g);
    if (!inst) return SPECV_E_HIP;
    if (hipEventCreateWithFlags(&e.done, hipEventDisableTiming) != hipSuccess) {
        destroy_entry(e);
        return SPECV_E_HIP;
    }
    if (gc.entries.size() >= kGraphCacheMax) {  // retire the least recently used entry
        auto lru = gc.entries.begin();
        for (auto i = gc.entries.begin(); i != gc.entries.end(); ++i)
            if (i->second.last_use < lru->second.last_use) lru = i;
        gc.retired.push_back(lru->second);
        gc.entries.erase(lru);
    }
    *out = &gc.entries.emplace(k, e).first->second;
    return SPECV_OK;
}

// The window itself: the cached step graph replayed W times, then the
// readback of the control block and the statistics.
static int run_window(const WindowKey& k, const StepLayout& lay, int W, void* host_readback, hipStream_t s) {
    specv_ctrl* ctrl = k.ctrl;
    specv_step_stats* stats = k.stats;
    void* workspace = k.workspace;
    GraphCache& gc = graph_cache();
    std::lock_guard<std::mutex> lock(gc.mu);
    reap_retired(gc);
    GraphEntry* entry = nullptr;
    int rc = window_graph(gc, k, lay, &entry);
    if (rc != SPECV_OK) return rc;
    entry->last_use = ++gc.clock;
    int32_t* wcounter = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + lay.wcounter);
    hipLaunchKernelGGL(window_begin_kernel, dim3(1), dim3(64), 0, s, wcounter);
    rc = launch_status();
    if (rc != SPECV_OK) return rc;
    for (int i = 0; i < W; i++)
        if (hipGraphLaunch(entry->exec, s) != hipSuccess) return SPECV_E_HIP;
    if (hipEventRecord(entry->done, s) != hipSuccess) return SPECV_E_HIP;
    if (host_readback) {
        char* hb = static_cast<char*>(host_readback);
        if (hipMemcpyAsync(hb, ctrl, sizeof(specv_ctrl), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipMemcpyAsync(hb + sizeof(specv_ctrl), stats, sizeof(specv_step_stats) * (size_t)W,
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return SPECV_E_HIP;
    }
    return SPECV_OK;
}

}  // namespace specv

extern "C" size_t spec_window_workspace(const specv_model* m, int32_t width) {
    return spec_step_workspace(m, width);
}

extern "C" int spec_window_run(const specv_model* m, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* ring,
                               int32_t ring_cap, const specv_drafter* d, int32_t width, int32_t W,
                               void* workspace, size_t workspace_bytes, void* host_readback, void* stream) {
    using namespace specv;
    const int vrc = validate_model(m);
    if (vrc != SPECV_OK) return vrc;
    if (width < 1 || width > 16 || W < 0 || W > 4096) return SPECV_E_SHAPE;
    if (width > 1 && m->vocab < 2) return SPECV_E_SHAPE;  // the drafter reduces modulo V - 1
    if (!ctrl || !stats) return SPECV_E_INVAL;
    if (ring && ring_cap < 1) return SPECV_E_INVAL;
    if (width > 1 && (!d || !d->reference || d->reference_len < 1 || !d->draws || d->draw_rows < 1))
        return SPECV_E_INVAL;
    if (!aligned(ctrl, 4) || !aligned(stats, 4) || !aligned(ring, 4)) return SPECV_E_ALIGN;
    const StepLayout lay = step_layout(m, width);
    if (!workspace || workspace_bytes < lay.total) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 256)) return SPECV_E_ALIGN;
    if (W == 0) return SPECV_OK;

    WindowKey k;
    std::memset(&k, 0, sizeof(k));
    k.model = *m;
    k.ctrl = ctrl;
    k.stats = stats;
    k.ring = ring;
    k.ring_cap = ring ? ring_cap : 0;
    k.width = width;
    k.drafter_kind = width > 1 ? kSynthetic : kRootOnly;
    if (k.drafter_kind == kSynthetic) {
        k.drafter = *d;
        k.drafter.reserved = 0;
    }
    k.workspace = workspace;
    return run_window(k, lay, W, host_readback, (hipStream_t)stream);
}

extern "C" size_t spec_window_cm_workspace(const specv_model* m, int32_t width, int32_t ring_cap,
                                           const specv_cm_params* p) {
    using namespace specv;
    if (validate_model(m) != SPECV_OK || width < 1 || width > 16 || ring_cap < 1 || ring_cap > (1 << 24) ||
        !cm_params_ok(p))
        return 0;
    return step_layout(m, width).total + cm_workspace_bytes(ring_cap, p);
}

extern "C" int spec_window_run_cm(const specv_model* m, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* ring,
                                  int32_t ring_cap, const specv_cm_params* p, int32_t width, int32_t W,
                                  void* workspace, size_t workspace_bytes, void* host_readback, void* stream) {
    using namespace specv;
    const int vrc = validate_model(m);
    if (vrc != SPECV_OK) return vrc;
    if (width < 1 || width > 16 || W < 0 || W > 4096 || ring_cap > (1 << 24)) return SPECV_E_SHAPE;
    if (!ctrl || !stats || !ring || ring_cap < 1 || !p || !cm_params_ok(p)) return SPECV_E_INVAL;
    if (!aligned(ctrl, 4) || !aligned(stats, 4) || !aligned(ring, 4)) return SPECV_E_ALIGN;
    const StepLayout lay = step_layout(m, width);
    if (!workspace || workspace_bytes < lay.total + cm_workspace_bytes(ring_cap, p)) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 256)) return SPECV_E_ALIGN;
    if (W == 0) return SPECV_OK;

    WindowKey k;
    std::memset(&k, 0, sizeof(k));
    k.model = *m;
    k.ctrl = ctrl;
    k.stats = stats;
    k.ring = ring;
    k.ring_cap = ring_cap;
    k.width = width;
    k.drafter_kind = kContextMixing;
    k.cm = *p;
    k.workspace = workspace;
    return run_window(k, lay, W, host_readback, (hipStream_t)stream);
}

