// Tree-masked forward of one verification step (GPU-Resident Speculative
// Decoding for In-Browser LLM Inference with WebGPU, Small-Batch
// Verification Kernels and GPU-Resident Speculation Loop) for a
// Qwen2.5-shaped decoder in the W4A8 format, plus the step that follows it
// (argmax, acceptance, compaction).
//
// All step kernels read the committed length, the node count and the done
// flag from the device control block when they run, so one enqueued (or
// graph-captured) step serves every step of a window.
//
// Arithmetic rules shared with every kernel of the library: single IEEE fp32
// operations in the written order, no contraction; every sum over a vector
// uses the 16-slot order (slot s takes indices s, s+16, ... in order, then
// the slots are added as a binary tree in index order). The xor butterfly
// over 16 lanes used below computes exactly that tree: after level w every
// aligned block of 2w lanes holds its block sum in every lane.
#include <cmath>
#include <cstring>

#include "common.h"
#include "internal.h"

namespace specv {


// Value of another lane of the same 16-lane row, by a DPP control: 0xB1 and
// 0x4E are the quad permutes of lane ^ 1 and lane ^ 2, 0x141 mirrors each
// half row (l <-> 7 - l), 0x140 the whole row (l <-> 15 - l).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    const int x = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false));
}

// Sum of one value per lane over 16 aligned lanes, in the tree order. After
// the xor-1 and xor-2 levels every lane of a quad holds the quad's sum, so the
// half-row mirror brings each lane the other quad's sum (level w = 4) and the
// row mirror the other half's (w = 8): every lane ends with the same bits,
// the adjacent-pair tree.
__device__ __forceinline__ float tree16(float v) {
    v = v + dpp_f32<0xB1>(v);
    v = v + dpp_f32<0x4E>(v);
    v = v + dpp_f32<0x141>(v);
    v = v + dpp_f32<0x140>(v);
    return v;
}

// Max over 16 aligned lanes (order-free), same exchanges as tree16.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return v;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
// a * (float)h as one fused multiply-add with a +0 addend: the rounded
// product itself (a zero product comes out +0, which a sum that starts at +0
// cannot tell from -0), taken by v_fma_mix_f32 straight from the half of a
// packed register, without a conversion.
__device__ __forceinline__ float mul_f16(float a, uint16_t h) { return __builtin_fmaf(a, f16_to_f32(h), 0.0f); }
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}

constexpr int kFwdThreads = 256;   // embedding and attention-chunk workgroups
constexpr int kRowThreads = 1024;  // row kernels: norms, SiLU, attention merge
// RMSNorm rows are produced by the linear that consumes them up to this many
// tokens (every workgroup recomputing them all): rows of up to 1024 values
// kept in registers, longer rows through LDS.
constexpr int kNormFuseMaxT = 8;
constexpr int kNormFuseMaxTLong = 4;
constexpr int kRowRegs = 4;        // float4 chunks per thread: rows up to 16384 values
constexpr int kMergeRegs = 8;      // values per thread in the merge: rows up to 8192
constexpr int kMaxNodes = 16;

// Block-wide max of non-negative values over kRowThreads threads (order-free):
// each 16-lane row by DPP, the wave's four rows read as scalars, then the
// waves' maxima through LDS.
__device__ __forceinline__ float block_max(float a, float* red) {
    a = max16(a);
    const int b = __builtin_bit_cast(int, a);
    a = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
              fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kRowThreads / 64; w++) r = fmaxf(r, red[w]);
    return r;
}

// Per-token int8 quantisation of a row held in registers (absmax scale,
// codes rounded to nearest-even, symmetric 127). Thread t holds, for r < R,
// the V values at columns V*(t + r*kRowThreads) + e.
template <int R, int V>
__device__ void quantize_regs(const float (&y)[R][V], int K, int8_t* __restrict__ xrow, float* __restrict__ xs_i,
                              float* red) {
    const int tid = threadIdx.x;
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < R; r++)
        if (V * (tid + r * kRowThreads) < K)
#pragma unroll
            for (int e = 0; e < V; e++) a = fmaxf(a, fabsf(y[r][e]));
    a = block_max(a, red);
    const QuantScale qs = quant_scale(a);
    if (tid == 0) *xs_i = a == 0.0f ? 0.0f : a / 127.0f;
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int c0 = V * (tid + r * kRowThreads);
        if (c0 >= K) continue;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < V; e++) packed |= (uint32_t)(uint8_t)(int8_t)(int)quant_code(y[r][e], qs) << (8 * e);
        if (V == 4)
            *reinterpret_cast<uint32_t*>(xrow + c0) = packed;
        else
            xrow[c0] = (int8_t)(packed & 0xff);
    }
}

// Positions per slot row of the RMSNorm kernel's transposed squares (H/16
// rounded up to whole blocks of 64, the tail zero), and the row's stride in
// floats: 4 more, so the 16 summing lanes read distinct banks, except for the
// longest rows (H = 16384), whose 16 rows then fill 64 KB exactly.
inline __host__ __device__ int norm_slot_positions(int H) { return ((H >> 4) + 63) & ~63; }
inline __host__ __device__ int norm_slot_stride(int H) {
    const int n = norm_slot_positions(H);
    return n < 1024 ? n + 4 : n;
}

// Rows of nodes past the live count quantise to zero, so the linears that
// follow produce exact zeros for them. K is a multiple of 4.
__device__ void zero_row(int8_t* xrow, float* xs_i, int K) {
    if (threadIdx.x == 0) *xs_i = 0.0f;
    for (int c = threadIdx.x; c < K / 4; c += blockDim.x) reinterpret_cast<uint32_t*>(xrow)[c] = 0;
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Tree info of a step, written once by the embedding kernel: depth[i], then
// anc[i][t] = the node at depth t on the path from the root to node i
// (anc[i][depth[i]] = i). A node whose parent breaks the topological order
// counts as a root.
constexpr int kTreeInfoInts = kMaxNodes + kMaxNodes * kMaxNodes;
__device__ __forceinline__ const int32_t* tinfo_anc(const int32_t* tinfo, int i) {
    return tinfo + kMaxNodes + i * kMaxNodes;
}

// ---------------------------------------------------------------- kernels

// Embedding tied to the lm_head: h[i][k] = f32(scale[k/32][tok]) * code(tok, k)
// (exact: an 11-bit significand times a 4-bit integer).
__global__ __launch_bounds__(kFwdThreads) void embed_kernel(const int32_t* __restrict__ token,
                                                            const int32_t* __restrict__ parent,
                                                            const uint8_t* __restrict__ wlm,
                                                            const uint16_t* __restrict__ slm, int H, int V,
                                                            float* __restrict__ h, int32_t* __restrict__ tinfo,
                                                            const specv_ctrl* ctrl) {
    __shared__ int s_par[kMaxNodes];
    const int i = blockIdx.x;
    if (ctrl->done || i >= ctrl->n_nodes) return;
    if (threadIdx.x <= i) s_par[threadIdx.x] = parent[threadIdx.x];
    int tok = token[i];
    tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
    // row tok of the packed lm_head: tile tok / 16, row tok % 16 of each
    // group's 16-row chunk
    const size_t G = (size_t)(H >> 5);
    const size_t tbase = (size_t)(tok >> 4) * G * 16 + (size_t)(tok & 15);
    for (int k = threadIdx.x; k < H; k += kFwdThreads) {
        const size_t c = tbase + (size_t)(k >> 5) * 16;
        const uint8_t b = wlm[c * 16 + ((k & 31) >> 1)];
        const int code = ((k & 1) ? (b >> 4) : (b & 15)) - 8;
        h[(size_t)i * H + k] = f16_to_f32(slm[c]) * (float)code;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int d = 0;
        for (int x = i; x > 0;) {
            const int p = s_par[x];
            if (p < 0 || p >= x) break;
            x = p;
            d++;
        }
        tinfo[i] = d;
        int32_t* anc = tinfo + kMaxNodes + i * kMaxNodes;
        for (int t = d, x = i; t >= 0; t--) {
            anc[t] = x;
            const int p = s_par[x];
            x = (p >= 0 && p < x) ? p : 0;
        }
    }
}

// Optional residual (h += resid, written back), RMSNorm with weight w, then
// per-token int8 quantisation. RMSNorm: ss = R16(x*x), ms = ss / H,
// rs = 1 / sqrt(ms + eps), y = (x * rs) * w. Every global load of the row is
// issued before the first use, so the kernel pays one memory round trip.
__global__ __launch_bounds__(kRowThreads) void rmsnorm_quant_kernel(float* __restrict__ h,
                                                                    const float* __restrict__ resid,
                                                                    const float* __restrict__ w, int H,
                                                                    float eps, int8_t* __restrict__ xq,
                                                                    float* __restrict__ xs,
                                                                    const specv_ctrl* ctrl) {
    extern __shared__ __attribute__((aligned(16))) float sq[];  // squares transposed: 16 slot rows
    __shared__ float red[kRowThreads / 64];
    __shared__ float s_ss;
    const int i = blockIdx.x, tid = threadIdx.x, H4 = H / 4;
    const int sstride = norm_slot_stride(H);
    if (ctrl->done) return;
    if (i >= ctrl->n_nodes) {
        zero_row(xq + (size_t)i * H, xs + i, H);
        return;
    }
    float* hr = h + (size_t)i * H;
    const float* rr = resid ? resid + (size_t)i * H : nullptr;
    float4 xv[kRowRegs], rv[kRowRegs], wv[kRowRegs];
#pragma unroll
    for (int r = 0; r < kRowRegs; r++) {
        const int c = tid + r * kRowThreads;
        if (c < H4) {
            xv[r] = ld4(hr + 4 * c);
            wv[r] = ld4(w + 4 * c);
            if (rr) rv[r] = ld4(rr + 4 * c);
        }
    }
    float x[kRowRegs][4];
    const int npos = norm_slot_positions(H);
#pragma unroll
    for (int r = 0; r < kRowRegs; r++) {
        const int c = tid + r * kRowThreads;
        if (c >= 4 * npos) continue;
        if (c < H4) {
            x[r][0] = xv[r].x, x[r][1] = xv[r].y, x[r][2] = xv[r].z, x[r][3] = xv[r].w;
            if (rr) {
                x[r][0] = x[r][0] + rv[r].x, x[r][1] = x[r][1] + rv[r].y;
                x[r][2] = x[r][2] + rv[r].z, x[r][3] = x[r][3] + rv[r].w;
                *reinterpret_cast<float4*>(hr + 4 * c) = make_float4(x[r][0], x[r][1], x[r][2], x[r][3]);
            }
        } else {  // the zero tail of the slot rows
            x[r][0] = x[r][1] = x[r][2] = x[r][3] = 0.0f;
        }
        // input k = 4c + e sits at slot k mod 16, position k / 16 of the
        // slot's row of the transposed copy
        float* q = sq + (4 * c & 15) * sstride + (c >> 2);
        q[0] = x[r][0] * x[r][0];
        q[sstride] = x[r][1] * x[r][1];
        q[2 * sstride] = x[r][2] * x[r][2];
        q[3 * sstride] = x[r][3] * x[r][3];
    }
    __syncthreads();
    if (tid < 16) {  // slot tid: its row in increasing k, read 16 float4s at a time
        // (the zeros past H / 16 leave a sum of squares unchanged, bit for bit)
        const float* row = sq + tid * sstride;
        float acc = 0.0f;
        for (int b0 = 0; b0 < npos; b0 += 64) {
            float4 v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) v[u] = *reinterpret_cast<const float4*>(row + b0 + 4 * u);
#pragma unroll
            for (int u = 0; u < 16; u++) acc = (((acc + v[u].x) + v[u].y) + v[u].z) + v[u].w;
        }
        acc = tree16(acc);
        if (tid == 0) s_ss = acc;
    }
    __syncthreads();
    const float ms = s_ss / (float)H;
    const float rs = 1.0f / sqrtf(ms + eps);
    float y[kRowRegs][4];
#pragma unroll
    for (int r = 0; r < kRowRegs; r++) {
        y[r][0] = (x[r][0] * rs) * wv[r].x;
        y[r][1] = (x[r][1] * rs) * wv[r].y;
        y[r][2] = (x[r][2] * rs) * wv[r].z;
        y[r][3] = (x[r][3] * rs) * wv[r].w;
    }
    quantize_regs(y, H, xq + (size_t)i * H, xs + i, red);
}

// Quantisation of the rows z = silu(gate) * up [n][I] that the gate_up
// linear's epilogue wrote (for steps whose down projection does not
// quantise them in its own prologue).
__global__ __launch_bounds__(kRowThreads) void rows_quant_kernel(const float* __restrict__ zr, int I,
                                                                 int8_t* __restrict__ xq, float* __restrict__ xs,
                                                                 const specv_ctrl* ctrl) {
    __shared__ float red[kRowThreads / 64];
    const int i = blockIdx.x, tid = threadIdx.x, I4 = I / 4;
    if (ctrl->done) return;
    if (i >= ctrl->n_nodes) {
        zero_row(xq + (size_t)i * I, xs + i, I);
        return;
    }
    const float* row = zr + (size_t)i * I;
    float4 zv[kRowRegs];
#pragma unroll
    for (int r = 0; r < kRowRegs; r++) {
        const int c = tid + r * kRowThreads;
        if (c < I4) zv[r] = ld4(row + 4 * c);
    }
    float z[kRowRegs][4];
#pragma unroll
    for (int r = 0; r < kRowRegs; r++) {
        if (tid + r * kRowThreads >= I4) continue;
        z[r][0] = zv[r].x;
        z[r][1] = zv[r].y;
        z[r][2] = zv[r].z;
        z[r][3] = zv[r].w;
    }
    quantize_regs(z, I, xq + (size_t)i * I, xs + i, red);
}

constexpr int kAttnChunk = 256;   // logical positions per chunk
constexpr int kMaxHeadDim = 128;
constexpr int kMaxGroup = 16;     // query heads per KV head
// How the attention chunks hold the value rows, by the step's node count
// (measured on MI355X, 0.5B decoder, per window step):
// - at most kAttnVregMaxNodes nodes: each summing lane loads its value words
//   straight into registers (width 1: 838 -> 826 us); from two nodes the
//   narrower loads cost more (927 -> 935 us at width 2);
// - otherwise the rows are staged in LDS, padded by 8 halves per row;
// - from kAttnSwizzleMinNodes nodes, for head dims that are a multiple of 64,
//   unpadded with the 16-byte chunks of row p XOR-swizzled (chunk t stored
//   at t ^ ((p >> 1) & 7)). Rows are then 128 or 256 bytes, and the 16 rows
//   a 16-lane group reads at one column land on 16 distinct 4-bank offsets
//   of the 64 banks. The 32 KB of rows (against 36 KB) let 4 workgroups
//   share a CU instead of 3: width 8 1233 -> 1213 us, width 16 1646 ->
//   1582 us, but width 4 1026 -> 1043 us.
constexpr int kAttnVregMaxNodes = 1;
constexpr int kAttnSwizzleMinNodes = 8;

inline __host__ __device__ constexpr bool attn_swizzle_ok(int hd) { return hd % 64 == 0; }
// Row of the staged values, in fp16 elements.
inline __host__ __device__ constexpr int attn_vstride(int hd, bool swz) { return swz ? hd : hd + 8; }

inline size_t attn_lds_bytes(int hd, bool vreg, bool swz) {  // dynamic part: the staged value rows
    return vreg ? 0 : (size_t)2 * kAttnChunk * attn_vstride(hd, swz);
}

inline size_t merge_lds_bytes(int nh, int nchunk_max) { return (size_t)4 * nh * (nchunk_max + 1); }

// Rotate-half rotary position p of one head's pair (x_d, x_{d+h}), h = HD/2:
// x'_d = x_d c - x_{d+h} s, x'_{d+h} = x_{d+h} c + x_d s, with c, s the
// table's fp32 values for (p, d).
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float& ra, float& rb) {
    ra = a * c - b * s;
    rb = b * c + a * s;
}

// One chunk of the visible sequence of one node for one query head. Logical
// position j < L is cache row j; position L + t is the node's ancestor at
// depth t (the node itself last), whose key and value this step makes: the
// key rotated at position L + t and both rounded to fp16, exactly the row
// the step writes to the cache at physical row L + ancestor. The query of
// the node is rotated at position L + depth(i). The workgroup of chunk 0 and
// the first query head of each KV group writes node i's key and value rows
// to the caches (no workgroup of this launch reads them). For the head:
// s_j = R16_d(q_d * K_jd) * scale, m = max s_j, e_j = E(s_j - m),
// l = R16_j(e_j), o_d = R16_j(e_j * V_jd), sums over the chunk's positions
// in logical order. Output per (node, head, chunk): m, l, o[hd].
//
// One workgroup per (chunk, query head, node): the query heads that share a
// KV head read the same rows, which the L2 serves after the first; one head
// per workgroup keeps each workgroup's dependent chains short and gives the
// chip more of them. The grid is (query head, node, chunk), so workgroups
// are dispatched chunk by chunk: those of the chunks past a node's sequence,
// which only read the control block and exit, come last instead of taking
// slots between the working ones. Thread t owns position t of the chunk and its key row.
// For the value sums, lane s of 16-lane group q takes R16 slot s (positions
// s, s+16, ... in order) of columns 4q .. 4q+3 (and 64 + 4q .. for head dims
// above 64), and the group's butterfly adds the slots as the index-order
// tree. With VREG each lane loads the value words of its slot straight into
// registers; otherwise thread t also loads the value row of position t
// (16-byte loads) and stages it in LDS, padded or, with SWZ, swizzled. All
// three compute the same sums. The query is loaded first and committed rows right
// after it, so neither waits for the other; only the tree positions wait for
// the ancestor list.
template <int HD, bool VREG, bool SWZ>
__global__ __launch_bounds__(kFwdThreads) void attn_chunk_kernel(
    const float* __restrict__ qkv, const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ tinfo, int layer, int cap,
    int nh, int nkv, float scale, float* __restrict__ part, int nchunk_max, const specv_ctrl* ctrl) {
    constexpr int HALF = HD / 2;
    constexpr int NB = (HD + 63) / 64;  // column blocks of 64 (16 groups x 4 columns)
    const int hq = blockIdx.x, i = blockIdx.y, c = blockIdx.z, tid = threadIdx.x;
    const int depth_raw = tinfo[i];  // issued with the control loads (i < 16)
    if (ctrl->done || i >= ctrl->n_nodes) return;
    const int L = ctrl->committed_len;
    if (L + i >= cap) return;  // its rows were not written (no room left)
    const int depth = min(max(depth_raw, 0), i);  // depth <= i in a topological tree
    const int len = L + depth + 1;
    const int j0 = c * kAttnChunk;
    if (j0 >= len) return;
    const int cnt = len - j0 < kAttnChunk ? len - j0 : kAttnChunk;
    const int grp = nh / nkv, g = hq / grp;
    const int QKV = (nh + 2 * nkv) * HD;
    __shared__ int anc[kMaxNodes];
    __shared__ __attribute__((aligned(16))) uint16_t tk[kMaxNodes][HD];  // the ancestors' fp16 key rows
    __shared__ __attribute__((aligned(16))) uint16_t tv[kMaxNodes][HD];  // and value rows
    __shared__ float qs[HD];
    __shared__ float S[kAttnChunk];
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem);  // [256][VS] without VREG
    constexpr int VS = attn_vstride(HD, SWZ);
    static_assert(!SWZ || attn_swizzle_ok(HD), "the swizzle permutes 8 chunks of 16 bytes");

    const size_t plane = (((size_t)layer * nkv + g) * cap) * HD;
    if (tid < HALF) {  // the node's rotated query
        const size_t tp = (size_t)(L + depth) * HALF + tid;
        const float* src = qkv + (size_t)i * QKV + hq * HD;
        rope_pair(src[tid], src[tid + HALF], cos_t[tp], sin_t[tp], qs[tid], qs[tid + HALF]);
    } else if (c == 0 && hq % grp == 0 && tid < 2 * HALF) {  // the node's key and value rows to the caches
        const int d = tid - HALF;
        const size_t tp = (size_t)(L + depth) * HALF + d;
        const float* ks = qkv + (size_t)i * QKV + (nh + g) * HD;
        const float* vs = qkv + (size_t)i * QKV + (nh + nkv + g) * HD;
        float ra, rb;
        rope_pair(ks[d], ks[d + HALF], cos_t[tp], sin_t[tp], ra, rb);
        const size_t row = plane + (size_t)(L + i) * HD;
        kc[row + d] = f32_to_f16(ra);
        kc[row + d + HALF] = f32_to_f16(rb);
        vc[row + d] = f32_to_f16(vs[d]);
        vc[row + d + HALF] = f32_to_f16(vs[d + HALF]);
    }
    const bool live = tid < cnt;
    const int j = j0 + tid;
    v4i kr[HD / 8], vr[VREG ? 1 : HD / 8];
    const bool early = live && j < L;
    if (early) {
        const v4i* ksrc = reinterpret_cast<const v4i*>(kc + plane + (size_t)j * HD);
#pragma unroll
        for (int t = 0; t < HD / 8; t++) kr[t] = ksrc[t];
        if constexpr (!VREG) {
            const v4i* vsrc = reinterpret_cast<const v4i*>(vc + plane + (size_t)j * HD);
#pragma unroll
            for (int t = 0; t < HD / 8; t++) vr[t] = vsrc[t];
        }
    }
    // with VREG, the value words of this lane's slot: position s + 16k,
    // columns d0 .. d0+3
    const int s = tid & 15, q = tid >> 4;
    uint2 vv[VREG ? NB : 1][16];
    if constexpr (VREG) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int d0 = 64 * b + 4 * q;
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int jj = j0 + s + 16 * k;
                vv[b][k] = make_uint2(0u, 0u);
                if (d0 < HD && s + 16 * k < cnt && jj < L)
                    vv[b][k] = *reinterpret_cast<const uint2*>(vc + plane + (size_t)jj * HD + d0);
            }
        }
    }
    if (tid <= depth) anc[tid] = min(max(tinfo_anc(tinfo, i)[tid], 0), i);
    __syncthreads();
    if (j0 + cnt > L) {  // the chunk holds tree positions: their rows, made once into LDS
        // The ancestor at depth t has depth t itself (its own walk to the root
        // is the tail of the node's), so its rotary position is L + t.
        for (int w = tid; w < (depth + 1) * HALF; w += kFwdThreads) {
            const int t = w / HALF, d = w - t * HALF;
            const int a = anc[t];
            const float* ks = qkv + (size_t)a * QKV + (nh + g) * HD;
            const float* vs = qkv + (size_t)a * QKV + (nh + nkv + g) * HD;
            const size_t tp = (size_t)(L + t) * HALF + d;
            float ra, rb;
            rope_pair(ks[d], ks[d + HALF], cos_t[tp], sin_t[tp], ra, rb);
            tk[t][d] = f32_to_f16(ra);
            tk[t][d + HALF] = f32_to_f16(rb);
            tv[t][d] = f32_to_f16(vs[d]);
            tv[t][d + HALF] = f32_to_f16(vs[d + HALF]);
        }
        __syncthreads();
        if (live && !early) {
            const v4i* ksrc = reinterpret_cast<const v4i*>(&tk[j - L][0]);
#pragma unroll
            for (int t = 0; t < HD / 8; t++) kr[t] = ksrc[t];
            if constexpr (!VREG) {
                const v4i* vsrc = reinterpret_cast<const v4i*>(&tv[j - L][0]);
#pragma unroll
                for (int t = 0; t < HD / 8; t++) vr[t] = vsrc[t];
            }
        }
        if constexpr (VREG) {
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const int d0 = 64 * b + 4 * q;
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    const int jj = j0 + s + 16 * k;
                    if (d0 < HD && s + 16 * k < cnt && jj >= L)
                        vv[b][k] = *reinterpret_cast<const uint2*>(&tv[jj - L][d0]);
                }
            }
        }
    }
    // score of this thread's position
    float sc = -__builtin_inff();
    if (live) {
        float slot[16];
#pragma unroll
        for (int r = 0; r < 16; r++) slot[r] = 0.0f;
#pragma unroll
        for (int t = 0; t < HD / 8; t++) {
            if constexpr (!VREG)
                *reinterpret_cast<v4i*>(Vs + tid * VS + 8 * (SWZ ? t ^ ((tid >> 1) & 7) : t)) = vr[t];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t wd = (uint32_t)kr[t][e];
                const int d = 8 * t + 2 * e;
                slot[d & 15] = slot[d & 15] + mul_f16(qs[d], (uint16_t)(wd & 0xffff));
                slot[(d + 1) & 15] = slot[(d + 1) & 15] + mul_f16(qs[d + 1], (uint16_t)(wd >> 16));
            }
        }
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
            for (int r = 0; r < 16; r += 2 * w) slot[r] = slot[r] + slot[r + w];
        sc = slot[0] * scale;
    }
    S[tid] = sc;
    __syncthreads();
    // max over the chunk, taken by every 16-lane group for itself (order-free;
    // only +0/-0 ties can differ, and a difference against either gives the
    // same exp input up to its sign)
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 16; k++)
        if (s + 16 * k < cnt) m = fmaxf(m, S[s + 16 * k]);
    m = max16(m);
    __syncthreads();
    S[tid] = live ? det_exp(sc - m) : 0.0f;
    __syncthreads();

    // Lane s of group q owns R16 slot s (positions s, s+16, ... in order) of
    // l and of the columns 4q..4q+3 (group q + 16, ... for head dims above
    // 64), read as one 8-byte word per position; the group's butterfly adds
    // the slots as the index-order tree. Every group also sums l; group 0
    // stores it.
    float* o = part + (((size_t)i * nh + hq) * nchunk_max + c) * (HD + 2);
    float e[16];
#pragma unroll
    for (int k = 0; k < 16; k++) e[k] = S[s + 16 * k];
    float l = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; k++)
        if (s + 16 * k < cnt) l = l + e[k];
    l = tree16(l);
    if (tid == 0) {
        o[0] = m;
        o[1] = l;
    }
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int d0 = 64 * b + 4 * q;
        if (d0 >= HD) break;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const int p = s + 16 * k;
            if (p < cnt) {
                uint2 w;
                if constexpr (VREG)
                    w = vv[b][k];
                else
                    w = *reinterpret_cast<const uint2*>(
                        Vs + p * VS + (SWZ ? 8 * ((d0 >> 3) ^ ((p >> 1) & 7)) + (d0 & 7) : d0));
                acc[0] = acc[0] + mul_f16(e[k], (uint16_t)(w.x & 0xffff));
                acc[1] = acc[1] + mul_f16(e[k], (uint16_t)(w.x >> 16));
                acc[2] = acc[2] + mul_f16(e[k], (uint16_t)(w.y & 0xffff));
                acc[3] = acc[3] + mul_f16(e[k], (uint16_t)(w.y >> 16));
            }
        }
#pragma unroll
        for (int r = 0; r < 4; r++) acc[r] = tree16(acc[r]);
        if (s == 0)
#pragma unroll
            for (int r = 0; r < 4; r++) o[2 + d0 + r] = acc[r];  // rows of HD + 2 floats: no vector store
    }
}

// Attention of one node for all the query heads that share one KV head,
// over one chunk of its visible sequence, with the merge fused: one
// workgroup per (KV head g, node i, chunk c), so each value row is read and
// widened once for the group's heads ([P1] Small-Batch Verification
// Kernels). The workgroup's NT threads (1024, or 512 for wide trees) form
// NT / 256 sets of 256; with S sets, set k takes the group's heads k,
// k + S, ... (at most 8 / S), so the SIMDs of a CU share the heads'
// arithmetic. With nsplit = 2 (small trees, where the grid is short of
// workgroups) two workgroups share a (KV head, node, chunk), the first
// taking heads 0..3 and the second the rest, one head per set: the rows are
// read twice (the second time mostly from L2) and each set's chain of
// dependent arithmetic is halved. In a set, thread t owns position t of the chunk: its
// key row meets each of its heads' queries, s_{h,t} = R16_d(q_d * K_td) *
// scale; each head's chunk maximum is taken over the set's waves (order-free);
// e_{h,t} = E(s_{h,t} - m_h). For the value sums, lane s of the set's 16-lane
// group q owns R16 slot s (positions s, s+16, ... in order) of columns
// 4q .. 4q+3 (and 64 + 4q .. for head dims above 64) and of l, then the
// group's butterfly adds the slots as the index-order tree: exactly the sums
// of the per-head kernel. The partials (m, l, o) are stored agent-coherently;
// the workgroup that arrives last for node i (one counter per node, reset by
// that workgroup) merges every head's chunks, m = max_c m_c, w_c = E(m_c -
// m), l = R16_c(w_c * l_c), o_d = R16_c(w_c * o_cd), out_d = o_d / l, and
// quantises the node's attention row for the output projection. No
// workgroup waits for another. Nodes past the live count quantise to zero.
constexpr int kGrpThreads = 1024;
constexpr int kGrpSets = kGrpThreads / kFwdThreads;  // sets of 256 threads
constexpr int kGrpMaxHeads = 8;                        // query heads per KV head the grouped kernel takes
constexpr int kGrpMaxRow = kGrpThreads;                // attention row (heads x head dim) its merge takes
constexpr int kGrpMaxChunks = 32;                      // chunks per node its merge takes
constexpr int kGrpSplitMaxNodes = 4;                   // trees up to this size split a group's heads
// Trees from this size take workgroups of 512 threads (two sets, up to four
// heads each): two fit on a CU, so the up to 2 x 16 x 17 workgroups of a
// wide tree run in one wave instead of two. Measured on the 0.5B window, us
// per step at widths 8 / 16: 965 / 1230 with 1024 threads, 990 / 1164 with
// 512 (980 / 1252 with 512 threads and the heads split over two
// workgroups), so only trees of more than 8 nodes take them.
constexpr int kGrpHalfMinNodes = 9;

template <int HD, int NT, bool MIX>
__global__ __launch_bounds__(NT) void attn_group_kernel(
    const float* __restrict__ qkv, const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ tinfo, int layer, int cap,
    int nh, int nkv, int nsplit, float scale, float* __restrict__ part, int nchunk_max,
    uint32_t* __restrict__ arrivals, int8_t* __restrict__ xq, float* __restrict__ xs, const specv_ctrl* ctrl) {
    constexpr int HALF = HD / 2;
    constexpr int NB = (HD + 63) / 64;
    constexpr bool SWZ = attn_swizzle_ok(HD);
    constexpr int VS = attn_vstride(HD, SWZ);
    constexpr bool KF = HD <= 64;  // key row widened to fp32 registers once (more than one head per set)
    constexpr int SETS = NT / kFwdThreads;          // sets of 256 threads
    constexpr int SH = kGrpMaxHeads / SETS;          // heads per set, at most
    constexpr int EPT = (kGrpMaxRow + NT - 1) / NT;  // merge: attention row elements per thread
    const int g = blockIdx.x / nsplit, sp = blockIdx.x - g * nsplit;
    const int i = blockIdx.y, c = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int set = __builtin_amdgcn_readfirstlane(tid >> 8);  // uniform in a wave
    const int t8 = tid & 255;                                  // position / lane of the set
    const int depth_raw = tinfo[i];  // issued with the control loads (i < 16)
    if (ctrl->done) return;
    const int K = nh * HD;
    if (i >= ctrl->n_nodes) {
        if (g == 0 && c == 0) zero_row(xq + (size_t)i * K, xs + i, K);
        return;
    }
    const int L = ctrl->committed_len;
    if (L + i >= cap) return;  // its rows were not written (no room left)
    const int depth = min(max(depth_raw, 0), i);
    const int len = L + depth + 1;
    const int j0 = c * kAttnChunk;
    if (j0 >= len) return;
    const int cnt = len - j0 < kAttnChunk ? len - j0 : kAttnChunk;
    const int G = nh / nkv;
    const int hps = (G + nsplit * SETS - 1) / (nsplit * SETS);  // heads per set (1 or 2)
    const int hbase = sp * SETS * hps;                             // this workgroup's first head
    const int QKV = (nh + 2 * nkv) * HD;
    __shared__ int anc[kMaxNodes];
    __shared__ __attribute__((aligned(16))) uint16_t tk[kMaxNodes][HD];
    __shared__ __attribute__((aligned(16))) uint16_t tv[kMaxNodes][HD];
    __shared__ __attribute__((aligned(16))) float qs[kGrpMaxHeads][HD];
    // e of position s + 16k at Et[h][s][4 * ((k >> 2) ^ ((s >> 2) & 3)) + (k & 3)]: each lane s reads its
    // 16 values as four 16-byte words, and the 16 lanes of a group hit distinct banks
    __shared__ __attribute__((aligned(16))) float Et[kGrpMaxHeads][16][16];
    __shared__ float wmax[NT / 64][SH];
    __shared__ int s_last;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem);  // [256][VS] value rows, then the key rows; later the
                                                       // merge's weights

    const size_t plane = (((size_t)layer * nkv + g) * cap) * HD;
    // Committed rows first, coalesced: set 0 loads the chunk's key rows and
    // set 1 its value rows, consecutive lanes reading consecutive 16-byte
    // pieces of a row, every load issued (rows past the committed ones read
    // zeros); both are staged in LDS, swizzled or padded as the value rows.
    constexpr int CH = HD / 8;          // 16-byte pieces per row
    constexpr int RPP = kFwdThreads / CH;  // rows per pass of a set
    uint16_t* Ks = Vs + kAttnChunk * VS;
    const int ncommit = L > j0 ? (L - j0 < cnt ? L - j0 : cnt) : 0;  // committed rows of the chunk
    v4i stage[CH];
    if (set < 2) {
        const auto rkv = make_rsrc((set == 0 ? kc : vc) + plane, (uint32_t)((size_t)cap * HD * 2));
        const int piece = t8 % CH;
#pragma unroll
        for (int pass = 0; pass < CH; pass++) {
            const int row = pass * RPP + t8 / CH;
            const bool ok = row < ncommit;
            stage[pass] = load16(rkv, ((uint32_t)(j0 + row) * (uint32_t)(HD * 2) + 16u * (uint32_t)piece) |
                                          (ok ? 0u : kOOB));
        }
    }
    for (int w = tid; w < G * HALF; w += NT) {  // the group's rotated queries of node i
        const int h = w / HALF, d = w - h * HALF;
        const size_t tp = (size_t)(L + depth) * HALF + d;
        const float* src = qkv + (size_t)i * QKV + (g * G + h) * HD;
        rope_pair(src[d], src[d + HALF], cos_t[tp], sin_t[tp], qs[h][d], qs[h][d + HALF]);
    }
    if (c == 0 && sp == 0 && tid >= NT - HALF) {  // node i's key and value rows to the caches
        const int d = tid - (NT - HALF);
        const size_t tp = (size_t)(L + depth) * HALF + d;
        const float* ks = qkv + (size_t)i * QKV + (nh + g) * HD;
        const float* vsrc = qkv + (size_t)i * QKV + (nh + nkv + g) * HD;
        float ra, rb;
        rope_pair(ks[d], ks[d + HALF], cos_t[tp], sin_t[tp], ra, rb);
        const size_t row = plane + (size_t)(L + i) * HD;
        kc[row + d] = f32_to_f16(ra);
        kc[row + d + HALF] = f32_to_f16(rb);
        vc[row + d] = f32_to_f16(vsrc[d]);
        vc[row + d + HALF] = f32_to_f16(vsrc[d + HALF]);
    }
    if (tid <= depth) anc[tid] = min(max(tinfo_anc(tinfo, i)[tid], 0), i);
    if (set < 2) {
        uint16_t* dst = set == 0 ? Ks : Vs;
        const int piece = t8 % CH;
#pragma unroll
        for (int pass = 0; pass < CH; pass++) {
            const int row = pass * RPP + t8 / CH;
            if (row < ncommit)
                *reinterpret_cast<v4i*>(dst + row * VS + 8 * (SWZ ? piece ^ ((row >> 1) & 7) : piece)) = stage[pass];
        }
    }
    __syncthreads();
    if (j0 + cnt > L) {  // the chunk holds tree positions: their rows, made once into LDS
        // the ancestor at depth t has depth t itself, so its rotary position is L + t
        for (int w = tid; w < (depth + 1) * HALF; w += NT) {
            const int t = w / HALF, d = w - t * HALF;
            const int a = anc[t];
            const float* ks = qkv + (size_t)a * QKV + (nh + g) * HD;
            const float* vsrc = qkv + (size_t)a * QKV + (nh + nkv + g) * HD;
            const size_t tp = (size_t)(L + t) * HALF + d;
            float ra, rb;
            rope_pair(ks[d], ks[d + HALF], cos_t[tp], sin_t[tp], ra, rb);
            tk[t][d] = f32_to_f16(ra);
            tk[t][d + HALF] = f32_to_f16(rb);
            tv[t][d] = f32_to_f16(vsrc[d]);
            tv[t][d + HALF] = f32_to_f16(vsrc[d + HALF]);
        }
        __syncthreads();
        // positions L .. len-1 of the chunk take the ancestors' rows
        if (set < 2 && t8 >= ncommit && t8 < cnt) {
            const uint16_t* src = set == 0 ? &tk[j0 + t8 - L][0] : &tv[j0 + t8 - L][0];
            uint16_t* dst = set == 0 ? Ks : Vs;
#pragma unroll
            for (int t = 0; t < CH; t++)
                *reinterpret_cast<v4i*>(dst + t8 * VS + 8 * (SWZ ? t ^ ((t8 >> 1) & 7) : t)) =
                    *reinterpret_cast<const v4i*>(src + 8 * t);
        }
        __syncthreads();
    }
    const bool live = t8 < cnt;
    v4i kr[HD / 8];
    if (live) {
#pragma unroll
        for (int t = 0; t < CH; t++)
            kr[t] = *reinterpret_cast<const v4i*>(Ks + t8 * VS + 8 * (SWZ ? t ^ ((t8 >> 1) & 7) : t));
    }
    // scores of this thread's position for the set's heads h = hbase + set + 4u:
    // with one head per set (MIX, chosen by the host) each product comes
    // straight from the key row's fp16 halves (v_fma_mix_f32: the products
    // need no conversion); with more, the key row is widened to fp32 once
    // (rows of up to 64 values) and shared by the heads, which costs less
    // than mixed products for each head
    float sc[SH];
    if constexpr (MIX) {
#pragma unroll
        for (int u = 0; u < SH; u++) sc[u] = -__builtin_inff();
        const int h = hbase + set;
        if (hps >= 1 && h < G && live) {
            float slot[16];
#pragma unroll
            for (int r = 0; r < 16; r++) slot[r] = 0.0f;
#pragma unroll
            for (int t = 0; t < HD / 8; t++) {
                const float4 qa = *reinterpret_cast<const float4*>(&qs[h][8 * t]);
                const float4 qb = *reinterpret_cast<const float4*>(&qs[h][8 * t + 4]);
                const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int d = 8 * t + e;
                    slot[d & 15] =
                        slot[d & 15] + mul_f16(qv[e], (uint16_t)(((uint32_t)kr[t][e >> 1]) >> (16 * (e & 1))));
                }
            }
#pragma unroll
            for (int w = 1; w < 16; w <<= 1)
#pragma unroll
                for (int r = 0; r < 16; r += 2 * w) slot[r] = slot[r] + slot[r + w];
            sc[0] = slot[0] * scale;
        }
    } else {
        float kf[KF ? HD : 1];
        if constexpr (KF) {
#pragma unroll
            for (int t = 0; t < HD / 8; t++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t wd = (uint32_t)kr[t][e];
                    kf[8 * t + 2 * e] = f16_to_f32((uint16_t)(wd & 0xffff));
                    kf[8 * t + 2 * e + 1] = f16_to_f32((uint16_t)(wd >> 16));
                }
        }
#pragma unroll
        for (int u = 0; u < SH; u++) {
            const int h = hbase + set + SETS * u;
            sc[u] = -__builtin_inff();
            if (u >= hps || h >= G || !live) continue;
            float slot[16];
#pragma unroll
            for (int r = 0; r < 16; r++) slot[r] = 0.0f;
#pragma unroll
            for (int t = 0; t < HD / 8; t++) {
                const float4 qa = *reinterpret_cast<const float4*>(&qs[h][8 * t]);
                const float4 qb = *reinterpret_cast<const float4*>(&qs[h][8 * t + 4]);
                const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int d = 8 * t + e;
                    float kd;
                    if constexpr (KF)
                        kd = kf[d];
                    else
                        kd = f16_to_f32((uint16_t)(((uint32_t)kr[t][e >> 1]) >> (16 * (e & 1))));
                    slot[d & 15] = slot[d & 15] + qv[e] * kd;
                }
            }
#pragma unroll
            for (int w = 1; w < 16; w <<= 1)
#pragma unroll
                for (int r = 0; r < 16; r += 2 * w) slot[r] = slot[r] + slot[r + w];
            sc[u] = slot[0] * scale;
        }
    }
    // each head's maximum over the chunk (order-free): rows by DPP, the four
    // rows of a wave by lane reads, the set's four waves through LDS
#pragma unroll
    for (int u = 0; u < SH; u++) {
        const float m16 = max16(sc[u]);
        const int b = __builtin_bit_cast(int, m16);
        const float mw = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
        if (lane == 0) wmax[wave][u] = mw;
    }
    __syncthreads();
    float mh[SH];
#pragma unroll
    for (int u = 0; u < SH; u++) {
        const int h = hbase + set + SETS * u;
        const int w0 = 4 * set;
        mh[u] = fmaxf(fmaxf(wmax[w0][u], wmax[w0 + 1][u]), fmaxf(wmax[w0 + 2][u], wmax[w0 + 3][u]));
        const int es = t8 & 15, ek = t8 >> 4;
        if (u < hps && h < G) Et[h][es][4 * ((ek >> 2) ^ ((es >> 2) & 3)) + (ek & 3)] = live ? det_exp(sc[u] - mh[u]) : 0.0f;
    }
    __syncthreads();

    const int s = t8 & 15, q = t8 >> 4;
    const auto rp = make_rsrc(part, 0x7fffffffu);
    auto put = [&](float* at, float v) {  // agent-coherent store of a partial
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), rp, (uint32_t)((at - part) * 4), 0,
                                              kCachePolicySC1);
    };
    float* pnode = part + ((size_t)i * nh + (size_t)g * G) * nchunk_max * (HD + 2) + (size_t)c * (HD + 2);
    if constexpr (MIX) {  // one head: the products straight from the value rows' fp16 halves
        const int u = 0, h = hbase + set;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int d0 = 64 * b + 4 * q;
            if (d0 >= HD) break;
            if (h >= G) break;
            uint2 vw[16];
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int p = s + 16 * k;
                vw[k] = make_uint2(0u, 0u);
                if (p < cnt)
                    vw[k] = *reinterpret_cast<const uint2*>(
                        Vs + p * VS + (SWZ ? 8 * ((d0 >> 3) ^ ((p >> 1) & 7)) + (d0 & 7) : d0));
            }
            float e[16];
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) {
                const float4 ev = *reinterpret_cast<const float4*>(&Et[h][s][4 * (k4 ^ ((s >> 2) & 3))]);
                e[4 * k4] = ev.x;
                e[4 * k4 + 1] = ev.y;
                e[4 * k4 + 2] = ev.z;
                e[4 * k4 + 3] = ev.w;
            }
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            float l = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; k++) {
                acc[0] = acc[0] + mul_f16(e[k], (uint16_t)(vw[k].x & 0xffff));
                acc[1] = acc[1] + mul_f16(e[k], (uint16_t)(vw[k].x >> 16));
                acc[2] = acc[2] + mul_f16(e[k], (uint16_t)(vw[k].y & 0xffff));
                acc[3] = acc[3] + mul_f16(e[k], (uint16_t)(vw[k].y >> 16));
                if (b == 0) l = l + e[k];
            }
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = tree16(acc[r]);
            float* o = pnode + (size_t)h * nchunk_max * (HD + 2);
            if (s == 0) {
#pragma unroll
                for (int r = 0; r < 4; r++) put(o + 2 + d0 + r, acc[r]);
            }
            if (b == 0 && q == 0) {
                l = tree16(l);
                if (s == 0) {
                    put(o, mh[u]);
                    put(o + 1, l);
                }
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int d0 = 64 * b + 4 * q;
            if (d0 >= HD) break;
            float v[16][4];
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int p = s + 16 * k;
                uint2 w = make_uint2(0u, 0u);
                if (p < cnt)
                    w = *reinterpret_cast<const uint2*>(Vs + p * VS + (SWZ ? 8 * ((d0 >> 3) ^ ((p >> 1) & 7)) + (d0 & 7)
                                                                            : d0));
                v[k][0] = f16_to_f32((uint16_t)(w.x & 0xffff));
                v[k][1] = f16_to_f32((uint16_t)(w.x >> 16));
                v[k][2] = f16_to_f32((uint16_t)(w.y & 0xffff));
                v[k][3] = f16_to_f32((uint16_t)(w.y >> 16));
            }
#pragma unroll
            for (int u = 0; u < SH; u++) {
                const int h = hbase + set + SETS * u;
                if (u >= hps || h >= G) continue;
                float e[16];
#pragma unroll
                for (int k4 = 0; k4 < 4; k4++) {
                    const float4 ev = *reinterpret_cast<const float4*>(&Et[h][s][4 * (k4 ^ ((s >> 2) & 3))]);
                    e[4 * k4] = ev.x;
                    e[4 * k4 + 1] = ev.y;
                    e[4 * k4 + 2] = ev.z;
                    e[4 * k4 + 3] = ev.w;
                }
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                float l = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    acc[0] = acc[0] + e[k] * v[k][0];
                    acc[1] = acc[1] + e[k] * v[k][1];
                    acc[2] = acc[2] + e[k] * v[k][2];
                    acc[3] = acc[3] + e[k] * v[k][3];
                    if (b == 0) l = l + e[k];
                }
#pragma unroll
                for (int r = 0; r < 4; r++) acc[r] = tree16(acc[r]);
                float* o = pnode + (size_t)h * nchunk_max * (HD + 2);
                if (s == 0) {
#pragma unroll
                    for (int r = 0; r < 4; r++) put(o + 2 + d0 + r, acc[r]);
                }
                if (b == 0 && q == 0) {
                    l = tree16(l);
                    if (s == 0) {
                        put(o, mh[u]);
                        put(o + 1, l);
                    }
                }
            }
        }
    }
    // arrival: this workgroup's partials are complete before its count (the
    // memory clobber keeps the compiler from moving the stores past the wait)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int nch = (len + kAttnChunk - 1) / kAttnChunk;
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(&arrivals[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before + 1 == (uint32_t)(nkv * nsplit * nch);
        if (last) __hip_atomic_store(&arrivals[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;

    // The merge of node i, by the last workgroup. Every load is issued
    // unconditionally, 16 chunks at a time, in one batch per thread: chunks
    // past nch read as zeros (out-of-range offsets) and are masked by
    // selects, so they add +0, which leaves a slot (never -0) unchanged.
    // First the chunk weights of each head (16 lanes per head, chunks s and
    // s + 16), with the thread's own partial outputs already in flight; then
    // the element of the attention row this thread owns.
    const int stride = HD + 2;
    const uint32_t rec = (uint32_t)stride * 4u;  // one chunk's record, bytes
    const uint32_t node_off = (uint32_t)((size_t)i * nh * nchunk_max * stride) * 4u;
    auto get = [&](uint32_t byte_off, bool ok) {  // agent-coherent load of node i's partials
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rp, (node_off + byte_off) | (ok ? 0u : kOOB), 0, kCachePolicySC1));
    };
    float* wts = reinterpret_cast<float*>(smem);  // [nh][nchunk_max], then l[nh]
    float* lsum = wts + (size_t)nh * nchunk_max;
    // element e of this thread: idx = tid + NT e of the row, head idx / HD
    int eh[EPT];
    bool own[EPT];
    uint32_t ebase[EPT];
    float slot[EPT][16];
#pragma unroll
    for (int e = 0; e < EPT; e++) {
        const int idx = tid + NT * e;
        eh[e] = idx / HD;
        own[e] = idx < K;
        ebase[e] = (uint32_t)((size_t)eh[e] * nchunk_max * stride + 2 + (idx - eh[e] * HD)) * 4u;
#pragma unroll
        for (int sl = 0; sl < 16; sl++) slot[e][sl] = 0.0f;
    }
    for (int c0 = 0; c0 < nch; c0 += 16) {
        float ov[EPT][16];
#pragma unroll
        for (int e = 0; e < EPT; e++)
#pragma unroll
            for (int sl = 0; sl < 16; sl++)
                ov[e][sl] = get(ebase[e] + (uint32_t)(c0 + sl) * rec, own[e] && c0 + sl < nch);
        if (c0 == 0) {
            const int hw = tid >> 4, sw = tid & 15;  // 16 lanes per head
            if (hw < nh) {
                const uint32_t hbase = (uint32_t)((size_t)hw * nchunk_max * stride) * 4u;
                const float mr0 = get(hbase + (uint32_t)sw * rec, sw < nch);
                const float mr1 = get(hbase + (uint32_t)(sw + 16) * rec, sw + 16 < nch);
                const float l0 = get(hbase + (uint32_t)sw * rec + 4u, sw < nch);
                const float l1 = get(hbase + (uint32_t)(sw + 16) * rec + 4u, sw + 16 < nch);
                const float m0 = sw < nch ? mr0 : -__builtin_inff();
                const float m1 = sw + 16 < nch ? mr1 : -__builtin_inff();
                const float m = max16(fmaxf(m0, m1));
                const float w0 = det_exp(m0 - m), w1 = det_exp(m1 - m);
                if (sw < nch) wts[hw * nchunk_max + sw] = w0;
                if (sw + 16 < nch) wts[hw * nchunk_max + sw + 16] = w1;
                float acc = 0.0f;
                acc = acc + (sw < nch ? w0 * l0 : 0.0f);
                acc = acc + (sw + 16 < nch ? w1 * l1 : 0.0f);
                acc = tree16(acc);
                if (sw == 0) lsum[hw] = acc;
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < EPT; e++) {
            if (!own[e]) continue;
            const float* wh = wts + eh[e] * nchunk_max;
#pragma unroll
            for (int sl = 0; sl < 16; sl++) {
                const float wc = c0 + sl < nch ? wh[c0 + sl] : 0.0f;
                slot[e][sl] = slot[e][sl] + wc * ov[e][sl];
            }
        }
    }
    float y[EPT];
    float ya = 0.0f;
#pragma unroll
    for (int e = 0; e < EPT; e++) {
        y[e] = 0.0f;
        if (!own[e]) continue;
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
            for (int sl = 0; sl < 16; sl += 2 * w) slot[e][sl] = slot[e][sl] + slot[e][sl + w];
        y[e] = slot[e][0] / lsum[eh[e]];
        ya = fmaxf(ya, fabsf(y[e]));
    }
    {
        const float m16 = max16(ya);
        const int b = __builtin_bit_cast(int, m16);
        const float mw = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
        if (lane == 0) wmax[wave][0] = mw;
    }
    __syncthreads();
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) a = fmaxf(a, wmax[w][0]);
    const QuantScale qsc = quant_scale(a);
    if (tid == 0) xs[i] = a == 0.0f ? 0.0f : a / 127.0f;
#pragma unroll
    for (int e = 0; e < EPT; e++)
        if (own[e]) xq[(size_t)i * K + tid + NT * e] = (int8_t)(int)quant_code(y[e], qsc);
}

// Merge of the chunks of each head of node i: m = max_c m_c,
// w_c = E(m_c - m), l = R16_c(w_c * l_c), o_d = R16_c(w_c * o_cd),
// out_d = o_d / l; then the attention output row [nh*hd] is quantised for
// the output projection. The chunk weights are computed once per
// (head, chunk) by 16 lanes per head and shared through LDS.
__global__ __launch_bounds__(kRowThreads) void attn_merge_quant_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ tinfo, int nh, int hd, int nchunk_max,
    int8_t* __restrict__ xq, float* __restrict__ xs, const specv_ctrl* ctrl) {
    extern __shared__ float wts[];  // [nh][nchunk_max] chunk weights, then l[nh]
    __shared__ float red[kRowThreads / 64];
    const int i = blockIdx.x, tid = threadIdx.x;
    const int K = nh * hd;
    if (ctrl->done) return;
    if (i >= ctrl->n_nodes) {
        zero_row(xq + (size_t)i * K, xs + i, K);
        return;
    }
    float* lsum = wts + (size_t)nh * nchunk_max;
    const int len = ctrl->committed_len + min(max(tinfo[i], 0), i) + 1;
    const int nch_len = (len + kAttnChunk - 1) / kAttnChunk;
    const int nch = nch_len < nchunk_max ? nch_len : nchunk_max;
    const int stride = hd + 2;
    // the first 16 chunks of this thread's first column, loaded before the
    // chunk weights are known (columns past the first kRowThreads load theirs
    // after them)
    float ov0[16];
    {
        const int hh = tid / hd, d = tid - hh * hd;
        const float* ph = part + ((size_t)i * nh + hh) * nchunk_max * stride + 2 + d;
#pragma unroll
        for (int c = 0; c < 16; c++) ov0[c] = tid < K && c < nch ? ph[(size_t)c * stride] : 0.0f;
    }
    for (int hh = tid >> 4; hh < nh; hh += kRowThreads / 16) {
        const int s = tid & 15;
        const float* ph = part + ((size_t)i * nh + hh) * nchunk_max * stride;
        float m = -__builtin_inff();
        for (int c = s; c < nch; c += 16) m = fmaxf(m, ph[(size_t)c * stride]);
        m = max16(m);
        float acc = 0.0f;
        for (int c = s; c < nch; c += 16) {
            const float wc = det_exp(ph[(size_t)c * stride] - m);
            wts[hh * nchunk_max + c] = wc;
            acc = acc + wc * ph[(size_t)c * stride + 1];
        }
        acc = tree16(acc);
        if (s == 0) lsum[hh] = acc;
    }
    __syncthreads();
    float y[kMergeRegs][1];
#pragma unroll
    for (int r = 0; r < kMergeRegs; r++) {
        const int idx = tid + r * kRowThreads;
        y[r][0] = 0.0f;
        if (idx >= K) continue;
        const int hh = idx / hd, d = idx - hh * hd;
        const float* ph = part + ((size_t)i * nh + hh) * nchunk_max * stride + 2 + d;
        const float* wh = wts + hh * nchunk_max;
        float slot[16];
#pragma unroll
        for (int s = 0; s < 16; s++) slot[s] = 0.0f;
        for (int c0 = 0; c0 < nch; c0 += 16) {
            float ov[16];
#pragma unroll
            for (int s = 0; s < 16; s++)
                ov[s] = r == 0 && c0 == 0 ? ov0[s] : c0 + s < nch ? ph[(size_t)(c0 + s) * stride] : 0.0f;
#pragma unroll
            for (int s = 0; s < 16; s++)
                if (c0 + s < nch) slot[s] = slot[s] + wh[c0 + s] * ov[s];
        }
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
            for (int s = 0; s < 16; s += 2 * w) slot[s] = slot[s] + slot[s + w];
        y[r][0] = slot[0] / lsum[hh];
    }
    quantize_regs(y, K, xq + (size_t)i * K, xs + i, red);
}

// ---------------------------------------------------------------- host

static inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

StepLayout step_layout(const specv_model* m, int n) {
    StepLayout s{};
    const size_t H = m->hidden, I = m->inter, V = m->vocab;
    const size_t QKV = (size_t)(m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
    const size_t A = (size_t)m->n_heads * m->head_dim;
    const size_t xq_cols = std::max(std::max(H, I), A);
    const int nch = (m->kv_capacity + kAttnChunk - 1) / kAttnChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    s.nchunk_max = nch;
    s.h = take(4 * n * H);
    s.h2 = take(4 * n * H);  // the residual ping-pongs between h and h2 when the norms are fused
    s.delta = take(4 * n * H);
    s.xq = take(n * xq_cols);
    s.xs = take(4 * n);
    s.qkv = take(4 * n * QKV);
    s.attn = take(4 * (size_t)n * m->n_heads * nch * (m->head_dim + 2));
    s.gu = take(4 * n * 2 * I);
    s.logits = take(4 * n * V);
    s.argmax_part = take(std::max(tree_argmax_accept_workspace(V, n), (size_t)n * (((V + 15) / 16 + 31) / 32 * 32) * sizeof(Best)));
    s.tree = take(4 * 16 * 4);  // parent, token, argmax, path for up to 16 nodes
    s.tinfo = take(4 * kTreeInfoInts);  // depths and ancestor lists of the step's tree
    s.wcounter = take(4);
    s.arrivals = take(4 * kMaxNodes);  // per node: chunk workgroups of the attention that have finished
    size_t lin = 0;
    for (size_t Nk : {QKV, H, 2 * I}) lin = std::max(lin, w4a8_linear_workspace(n, (int)Nk, (int)H));
    lin = std::max(lin, w4a8_linear_workspace(n, (int)H, (int)A));
    lin = std::max(lin, w4a8_linear_workspace(n, (int)H, (int)I));
    lin = std::max(lin, w4a8_linear_workspace(n, (int)V, (int)H));
    s.linear = take(lin);
    s.linear_bytes = lin;
    s.total = off;
    return s;
}

int validate_model(const specv_model* m) {
    if (!m) return SPECV_E_INVAL;
    if (m->n_layers < 1 || m->hidden < 32 || m->hidden % 32 || m->n_heads < 1 || m->n_kv_heads < 1 ||
        m->n_heads % m->n_kv_heads || m->n_heads / m->n_kv_heads > kMaxGroup || m->head_dim < 16 ||
        m->head_dim % 16 || m->head_dim > kMaxHeadDim || (m->n_heads * m->head_dim) % 32 || m->inter < 32 ||
        m->inter % 32 || m->vocab < 1 || m->max_pos < 1 || m->kv_capacity < 1 || m->max_pos < m->kv_capacity ||
        !(m->eps >= 0.0f) || attn_lds_bytes(m->head_dim, false, false) > 150 * 1024 ||
        (size_t)std::max(m->hidden, m->inter) * 4 > 64 * 1024 ||
        (size_t)m->n_heads * m->head_dim > (size_t)kMergeRegs * kRowThreads ||
        merge_lds_bytes(m->n_heads, (m->kv_capacity + kAttnChunk - 1) / kAttnChunk) > 64 * 1024)
        return SPECV_E_SHAPE;
    if (!m->w_qkv || !m->s_qkv || !m->w_o || !m->s_o || !m->w_gu || !m->s_gu || !m->w_down || !m->s_down ||
        !m->norm_attn || !m->norm_mlp || !m->norm_final || !m->w_lm || !m->s_lm || !m->rope_cos ||
        !m->rope_sin || !m->k_cache || !m->v_cache)
        return SPECV_E_INVAL;
    if (!aligned(m->k_cache, 16) || !aligned(m->v_cache, 16) || !aligned(m->norm_attn, 16) ||
        !aligned(m->norm_mlp, 16) || !aligned(m->norm_final, 16))
        return SPECV_E_ALIGN;
    return SPECV_OK;
}

#define SPECV_TRY(expr)            \
    do {                           \
        const int rc_ = (expr);    \
        if (rc_ != SPECV_OK) return rc_; \
    } while (0)

template <int HD>
static int launch_attn_hd(bool vreg, bool swz, dim3 grid, size_t lds, hipStream_t s, const float* qkv,
                          const float* cos_t, const float* sin_t, uint16_t* kc, uint16_t* vc, const int32_t* tinfo,
                          int layer, int cap, int nh, int nkv, float scale, float* part, int nchunk_max,
                          const specv_ctrl* ctrl) {
    auto kernel = vreg  ? &attn_chunk_kernel<HD, true, false>
                  : swz ? &attn_chunk_kernel<HD, false, attn_swizzle_ok(HD)>
                        : &attn_chunk_kernel<HD, false, false>;
    static size_t enabled[2] = {64 * 1024, 64 * 1024};  // dynamic LDS above 64 KB is enabled per kernel
    size_t& en = enabled[swz ? 1 : 0];
    if (lds > en) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        en = lds;
    }
    hipLaunchKernelGGL(kernel, grid, dim3(kFwdThreads), lds, s, qkv, cos_t, sin_t, kc, vc, tinfo, layer, cap, nh,
                       nkv, scale, part, nchunk_max, ctrl);
    return launch_status();
}

// The grouped attention with the fused merge takes at most kGrpMaxHeads query
// heads per KV head and an attention row of at most kGrpMaxRow values.
static bool attn_grouped_ok(const specv_model* m) {
    return m->n_heads / m->n_kv_heads <= kGrpMaxHeads && m->n_heads * m->head_dim <= kGrpMaxRow &&
           (m->kv_capacity + kAttnChunk - 1) / kAttnChunk <= kGrpMaxChunks;
}

inline size_t attn_group_lds_bytes(int hd, int nh, int nchunk_max) {  // key and value rows, or the merge
    return std::max(2 * attn_lds_bytes(hd, false, attn_swizzle_ok(hd)), merge_lds_bytes(nh, nchunk_max));
}

template <int HD, int NT, bool MIX>
static int launch_attn_group_nt(dim3 grid, size_t lds, hipStream_t s, const float* qkv, const float* cos_t,
                                const float* sin_t, uint16_t* kc, uint16_t* vc, const int32_t* tinfo, int layer,
                                int cap, int nh, int nkv, int nsplit, float scale, float* part, int nchunk_max,
                                uint32_t* arrivals, int8_t* xq, float* xs, const specv_ctrl* ctrl) {
    auto kernel = &attn_group_kernel<HD, NT, MIX>;
    static size_t enabled = 64 * 1024;  // dynamic LDS above 64 KB is enabled per kernel
    if (lds > enabled) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        enabled = lds;
    }
    hipLaunchKernelGGL(kernel, grid, dim3(NT), lds, s, qkv, cos_t, sin_t, kc, vc, tinfo, layer, cap, nh, nkv, nsplit,
                       scale, part, nchunk_max, arrivals, xq, xs, ctrl);
    return launch_status();
}

template <int HD>
static int launch_attn_group_hd(int threads, dim3 grid, size_t lds, hipStream_t s, const float* qkv,
                                const float* cos_t, const float* sin_t, uint16_t* kc, uint16_t* vc,
                                const int32_t* tinfo, int layer, int cap, int nh, int nkv, int nsplit, float scale,
                                float* part, int nchunk_max, uint32_t* arrivals, int8_t* xq, float* xs,
                                const specv_ctrl* ctrl) {
    // one query head per set (the kernel's hps) takes the mixed-precision products
    const int sets = threads / kFwdThreads, G = nh / nkv;
    const bool mix = (G + nsplit * sets - 1) / (nsplit * sets) == 1;
#define SPECV_GRP(NTV, MIXV)                                                                                     \
    return launch_attn_group_nt<HD, NTV, MIXV>(grid, lds, s, qkv, cos_t, sin_t, kc, vc, tinfo, layer, cap, nh, nkv, \
                                               nsplit, scale, part, nchunk_max, arrivals, xq, xs, ctrl)
    if (threads == kGrpThreads / 2) {
        if (mix) SPECV_GRP(kGrpThreads / 2, true);
        SPECV_GRP(kGrpThreads / 2, false);
    }
    if (mix) SPECV_GRP(kGrpThreads, true);
    SPECV_GRP(kGrpThreads, false);
#undef SPECV_GRP
}

static int launch_attn_group(int hd, int threads, int nsplit, dim3 grid, hipStream_t s, const float* qkv,
                             const float* cos_t, const float* sin_t, uint16_t* kc, uint16_t* vc,
                             const int32_t* tinfo, int layer, int cap, int nh, int nkv, float scale, float* part,
                             int nchunk_max, uint32_t* arrivals, int8_t* xq, float* xs, const specv_ctrl* ctrl) {
    const size_t lds = attn_group_lds_bytes(hd, nh, nchunk_max);
    switch (hd) {
#define SPECV_ATTN(HDV)                                                                                           \
    case HDV:                                                                                                     \
        return launch_attn_group_hd<HDV>(threads, grid, lds, s, qkv, cos_t, sin_t, kc, vc, tinfo, layer, cap, nh, \
                                         nkv, nsplit, scale, part, nchunk_max, arrivals, xq, xs, ctrl);
        SPECV_ATTN(16) SPECV_ATTN(32) SPECV_ATTN(48) SPECV_ATTN(64)
        SPECV_ATTN(80) SPECV_ATTN(96) SPECV_ATTN(112) SPECV_ATTN(128)
#undef SPECV_ATTN
        default: return SPECV_E_SHAPE;
    }
}

static int launch_attn_chunk(int hd, dim3 grid, hipStream_t s, const float* qkv, const float* cos_t,
                             const float* sin_t, uint16_t* kc, uint16_t* vc, const int32_t* tinfo, int layer,
                             int cap, int nh, int nkv, float scale, float* part, int nchunk_max,
                             const specv_ctrl* ctrl) {
    const bool vreg = (int)grid.y <= kAttnVregMaxNodes;
    const bool swz = !vreg && (int)grid.y >= kAttnSwizzleMinNodes && attn_swizzle_ok(hd);
    const size_t lds = attn_lds_bytes(hd, vreg, swz);
    switch (hd) {
#define SPECV_ATTN(HDV) \
    case HDV:           \
        return launch_attn_hd<HDV>(vreg, swz, grid, lds, s, qkv, cos_t, sin_t, kc, vc, tinfo, layer, cap, nh, nkv, \
                                   scale, part, nchunk_max, ctrl);
        SPECV_ATTN(16) SPECV_ATTN(32) SPECV_ATTN(48) SPECV_ATTN(64)
        SPECV_ATTN(80) SPECV_ATTN(96) SPECV_ATTN(112) SPECV_ATTN(128)
#undef SPECV_ATTN
        default: return SPECV_E_SHAPE;
    }
}

int enqueue_forward(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                    Best* amax, specv_ctrl* ctrl, char* ws, const StepLayout& lay, hipStream_t s) {
    const int H = m->hidden, I = m->inter, V = m->vocab, nh = m->n_heads, nkv = m->n_kv_heads, hd = m->head_dim;
    const int QKV = (nh + 2 * nkv) * hd, A = nh * hd, cap = m->kv_capacity;
    float* h = reinterpret_cast<float*>(ws + lay.h);
    float* h2 = reinterpret_cast<float*>(ws + lay.h2);
    float* delta = reinterpret_cast<float*>(ws + lay.delta);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + lay.xq);
    float* xs = reinterpret_cast<float*>(ws + lay.xs);
    float* qkv = reinterpret_cast<float*>(ws + lay.qkv);
    float* attn = reinterpret_cast<float*>(ws + lay.attn);
    float* gu = reinterpret_cast<float*>(ws + lay.gu);
    int32_t* tinfo = reinterpret_cast<int32_t*>(ws + lay.tinfo);
    void* lin = lay.linear_bytes ? ws + lay.linear : nullptr;
    const size_t linb = lay.linear_bytes;
    const float scale = (float)(1.0 / std::sqrt((double)hd));

    hipLaunchKernelGGL(embed_kernel, dim3(n), dim3(kFwdThreads), 0, s, token, parent, m->w_lm, m->s_lm, H, V, h,
                       tinfo, ctrl);
    SPECV_TRY(launch_status());
    // RMSNorm (of h, or of h + resid with the sum kept as the new residual)
    // and the linear that consumes it: one fused launch when the linear can
    // produce its rows, else the row kernel and the linear. Fused, the
    // residual alternates between h and h2.
    float* hcur = h;
    auto norm_linear = [&](const float* resid, const float* w, const uint8_t* wq, const uint16_t* ws_,
                           float* y, Best* am, int N, bool keep, int epi) -> int {
        if (n <= (H <= 1024 ? kNormFuseMaxT : kNormFuseMaxTLong) && linear_fused_supported(kProdNorm, n, H)) {
            float* hnext = !resid || !keep ? nullptr : (hcur == h ? h2 : h);
            ProdArgs pa{hcur, resid, w, hnext, m->eps, 0, ctrl, epi};
            const int rc = linear_enqueue_fused(kProdNorm, pa, wq, ws_, y, am, n, N, H, s);
            if (hnext) hcur = hnext;
            return rc;
        }
        hipLaunchKernelGGL(rmsnorm_quant_kernel, dim3(n), dim3(kRowThreads),
                           (size_t)16 * norm_slot_stride(H) * sizeof(float), s, hcur, resid, w,
                           H, m->eps, xq, xs, ctrl);
        SPECV_TRY(launch_status());
        return linear_enqueue(wq, ws_, xq, xs, y, am, n, N, H, lin, s, epi);
    };
    // The gate_up epilogue writes z = silu(gate) * up (its rows alternate in
    // blocks of 8 gate and 8 up rows); the down projection quantises z in
    // its own prologue while that fits, else a row kernel does.
    const bool fuse_rows = linear_fused_supported(kProdRows, n, I);
    const bool grouped = attn_grouped_ok(m);
    // small trees leave the grid short of workgroups: split each group's heads over two
    // wide trees: half-size workgroups (the merge's chunk weights take 16 lanes per head)
    const bool half = n >= kGrpHalfMinNodes && nh * 16 <= kGrpThreads / 2;
    const int grp_threads = half ? kGrpThreads / 2 : kGrpThreads;
    const int nsplit = !half && nh / nkv > kGrpSets && n <= kGrpSplitMaxNodes ? 2 : 1;
    uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + lay.arrivals);
    for (int l = 0; l < m->n_layers; l++) {
        // each layer's matrices in the packed tile layout, one after another
        const uint8_t* wqkv = m->w_qkv + (size_t)l * packed_weight_bytes(QKV, H);
        const uint16_t* sqkv = m->s_qkv + (size_t)l * packed_scale_bytes(QKV, H) / 2;
        const uint8_t* wo = m->w_o + (size_t)l * packed_weight_bytes(H, A);
        const uint16_t* so = m->s_o + (size_t)l * packed_scale_bytes(H, A) / 2;
        const uint8_t* wgu = m->w_gu + (size_t)l * packed_weight_bytes(2 * I, H);
        const uint16_t* sgu = m->s_gu + (size_t)l * packed_scale_bytes(2 * I, H) / 2;
        const uint8_t* wd = m->w_down + (size_t)l * packed_weight_bytes(H, I);
        const uint16_t* sd = m->s_down + (size_t)l * packed_scale_bytes(H, I) / 2;

        SPECV_TRY(norm_linear(l == 0 ? nullptr : delta, m->norm_attn + (size_t)l * H, wqkv, sqkv, qkv, nullptr, QKV,
                              true, kEpiPlain));
        if (grouped) {  // chunks of every head of a KV group, the merge by the last workgroup of each node
            SPECV_TRY(launch_attn_group(hd, grp_threads, nsplit, dim3(nkv * nsplit, n, lay.nchunk_max), s, qkv,
                                        m->rope_cos, m->rope_sin, m->k_cache, m->v_cache, tinfo, l, cap, nh, nkv,
                                        scale, attn, lay.nchunk_max, arrivals, xq, xs, ctrl));
        } else {
            SPECV_TRY(launch_attn_chunk(hd, dim3(nh, n, lay.nchunk_max), s, qkv, m->rope_cos, m->rope_sin,
                                        m->k_cache, m->v_cache, tinfo, l, cap, nh, nkv, scale, attn, lay.nchunk_max,
                                        ctrl));
            hipLaunchKernelGGL(attn_merge_quant_kernel, dim3(n), dim3(kRowThreads),
                               merge_lds_bytes(nh, lay.nchunk_max), s, attn, tinfo, nh, hd, lay.nchunk_max, xq, xs,
                               ctrl);
            SPECV_TRY(launch_status());
        }
        SPECV_TRY(w4a8_linear_T(wo, so, xq, xs, delta, n, H, A, lin, linb, s));
        SPECV_TRY(norm_linear(delta, m->norm_mlp + (size_t)l * H, wgu, sgu, gu, nullptr, 2 * I, true,
                              kEpiSiluPairs));
        if (fuse_rows) {
            ProdArgs pa{gu, nullptr, nullptr, nullptr, 0.0f, 0, ctrl, kEpiPlain};
            SPECV_TRY(linear_enqueue_fused(kProdRows, pa, wd, sd, delta, nullptr, n, H, I, s));
        } else {
            hipLaunchKernelGGL(rows_quant_kernel, dim3(n), dim3(kRowThreads), 0, s, gu, I, xq, xs, ctrl);
            SPECV_TRY(launch_status());
            SPECV_TRY(w4a8_linear_T(wd, sd, xq, xs, delta, n, H, I, lin, linb, s));
        }
    }
    // the residual is not needed after the final norm
    return norm_linear(delta, m->norm_final, m->w_lm, m->s_lm, logits, amax, V, false, kEpiPlain);
}

int enqueue_step(const specv_model* m, int n, const int32_t* parent, const int32_t* token, float* logits,
                 int32_t* argmax, int32_t* path, specv_ctrl* ctrl, specv_step_stats* stats, int32_t* wcounter,
                 int32_t* ring, int32_t ring_cap, char* ws, const StepLayout& lay, hipStream_t s) {
    // The lm_head's argmax epilogue reduces each workgroup's rows to one
    // (max, lowest index) pair per node, so the logits are written only when
    // the caller asks for them; acceptance finishes from the pairs.
    if (linear_argmax_supported(n, m->vocab, m->hidden)) {
        Best* part = reinterpret_cast<Best*>(ws + lay.argmax_part);
        SPECV_TRY(enqueue_forward(m, n, parent, token, logits, part, ctrl, ws, lay, s));
        SPECV_TRY(enqueue_accept(part, linear_argmax_chunks(n, m->vocab, m->hidden), nullptr, n, parent, token,
                                 argmax, path, ctrl, stats, wcounter, ring, ring_cap, s));
    } else {
        float* lg = logits ? logits : reinterpret_cast<float*>(ws + lay.logits);
        SPECV_TRY(enqueue_forward(m, n, parent, token, lg, nullptr, ctrl, ws, lay, s));
        SPECV_TRY(enqueue_argmax_accept(lg, m->vocab, n, parent, token, argmax, path, ctrl, stats, wcounter, ring,
                                        ring_cap, ws + lay.argmax_part, s));
    }
    return kv_compact(m->k_cache, m->v_cache, m->n_layers, m->n_kv_heads, m->kv_capacity, m->head_dim, path, ctrl,
                      s);
}

}  // namespace specv

extern "C" int specv_rope_table(float* cos_host, float* sin_host, int32_t max_pos, int32_t head_dim,
                                double theta) {
    if (!cos_host || !sin_host) return SPECV_E_INVAL;
    if (max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0)) return SPECV_E_SHAPE;
    const int half = head_dim / 2;
    for (int p = 0; p < max_pos; p++)
        for (int i = 0; i < half; i++) {
            const double a = (double)p * std::pow(theta, -2.0 * i / head_dim);
            cos_host[(size_t)p * half + i] = (float)std::cos(a);
            sin_host[(size_t)p * half + i] = (float)std::sin(a);
        }
    return SPECV_OK;
}

extern "C" size_t spec_step_workspace(const specv_model* m, int32_t n_max) {
    using namespace specv;
    if (validate_model(m) != SPECV_OK || n_max < 1 || n_max > 16) return 0;
    return step_layout(m, n_max).total;
}

extern "C" int spec_tree_step(const specv_model* m, specv_ctrl* ctrl, const int32_t* parent,
                              const int32_t* token, int32_t n_max, float* logits, int32_t* argmax,
                              int32_t* path, specv_step_stats* stats, int32_t* ring, int32_t ring_cap,
                              void* workspace, size_t workspace_bytes, void* stream) {
    using namespace specv;
    SPECV_TRY(validate_model(m));
    if (n_max < 1 || n_max > 16) return SPECV_E_SHAPE;
    if (!ctrl || !parent || !token || !argmax || !path) return SPECV_E_INVAL;
    if (ring && ring_cap < 1) return SPECV_E_INVAL;
    if (!aligned(ctrl, 4) || !aligned(parent, 4) || !aligned(token, 4) || !aligned(logits, 16) ||
        !aligned(argmax, 4) || !aligned(path, 4))
        return SPECV_E_ALIGN;
    const StepLayout lay = step_layout(m, n_max);
    if (!workspace || workspace_bytes < lay.total) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 256)) return SPECV_E_ALIGN;
    return enqueue_step(m, n_max, parent, token, logits, argmax, path, ctrl, stats, nullptr, ring, ring_cap,
                        static_cast<char*>(workspace), lay, (hipStream_t)stream);
}
