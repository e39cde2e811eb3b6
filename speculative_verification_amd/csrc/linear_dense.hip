// W4A8 linear for 17..32 tokens with dense integer matrix products.
//
// Same operation and order as the streaming kernel (GPU-Resident Speculative
// Decoding for In-Browser LLM Inference with WebGPU, Small-Batch
// Verification Kernels: token buckets up to 32 run the same integer
// kernels):
//   d[t][n][g] = sum_{k in group g} q(n,k) * xq[t][k]    exact int32
//   p_g        = f32(scale[g][n]) * f32(d)                one rounding
//   y[t][n]    = xs[t] * R16(p_0 .. p_{G-1})              fixed order
// R16: slot s accumulates groups s, s+16, s+32, ... in increasing g from +0;
// the 16 slots are added as a binary tree in index order.
//
// With 32 tokens the block-diagonal 16x16x64 form of the streaming kernel
// spends three quarters of every matrix instruction on zeros and reads as
// many activation operands as weights. Here each v_mfma_i32_16x16x32_i8 is
// dense: 16 tokens x 16 rows x the 32 inputs of one group, so one
// instruction per (16-row tile, group, 16-token tile).
//
// Work decomposition. A workgroup of 16 waves walks 16-row tiles b, b + nwg,
// ...; wave s owns R16 slot s, so it takes the groups s, s + 16, ... of every
// tile in increasing order (iteration j: group 16j + s), and the slot's
// running sum is the wave's own accumulator. Lane (r, q) (r = lane % 16,
// q = lane / 16) loads word q (inputs 8q .. 8q+7) of row r's 16-byte chunk
// of the group: the B operand of row r, k-quarter q. Its A operands, token
// (16tt + r)'s same 8 inputs, are loaded once per launch and stay in
// registers for every tile (JT iterations per tile, at most kDenseMaxJ). The
// product for row r lands in lane (r, q) itself, tokens 16tt + 4q + i, so the
// lane's own scale applies. Each iteration's weights are replaced, as they
// are consumed, by the same iteration's of the tile LA ahead (two tiles in
// flight up to 8 iterations per tile, else one). At the end of a tile the
// 16 slot sums of each (token, row) meet in LDS and are added as the
// index-order tree.
//
// Nibble decode as in the streaming kernel: a word of 8 codes u = q + 8
// becomes two int8 words of 16q (inputs 0, 2, 4, 6, then 1, 3, 5, 7), and the
// activation bytes of each 8-input chunk are put in the same order, so the
// products come out as 16d (exact) and the scale is pre-divided by 16
// (exact).
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kDenseThreads = 1024;  // 16 waves: one R16 slot each
constexpr int kDenseMaxJ = 10;       // iterations per tile whose activation operands stay in registers
constexpr int kDenseTokens = 32;
// Tiles of weights in flight for up to 8 iterations per tile (measured on
// MI355X at 32 tokens: three were no faster than two, and four spill).
constexpr int kDenseLookahead = 2;
// Passes of the streamed kernel whose activation and weight loads are in
// flight (measured, the 14336-input down projection at 32 tokens: 21.0,
// 21.4 and 22.8 us per launch with 2, 3 and 4).
constexpr int kDensePassAhead = 2;

// 8 activation codes (inputs 0..7) in the even-then-odd order of the decode.
__device__ __forceinline__ long even_odd8(uint64_t raw) {
    const uint32_t a0 = (uint32_t)raw, a1 = (uint32_t)(raw >> 32);
    const uint32_t ev = __builtin_amdgcn_perm(a1, a0, 0x06040200u);
    const uint32_t od = __builtin_amdgcn_perm(a1, a0, 0x07050301u);
    return (long)((uint64_t)ev | ((uint64_t)od << 32));
}

// The word's 8 codes as int8 values 16q, evens then odds.
__device__ __forceinline__ long decode_word(uint32_t W) {
    const uint32_t ev = ((W << 4) ^ 0x80808080u) & 0xF0F0F0F0u;
    const uint32_t od = (W ^ 0x80808080u) & 0xF0F0F0F0u;
    return (long)((uint64_t)ev | ((uint64_t)od << 32));
}

// Activation staging: chunks of kStageGroups groups x 32 tokens, 32-byte
// pieces at (group * 33 + token) * 32 (the padding spreads a wave's
// 16-byte writes over the banks).
constexpr int kStageGroups = 32;
constexpr int kStageBytes = kStageGroups * 33 * 32;

// Bias of the integer products: the matrix instruction adds it as C, so
// the int32 result read as fp32 is exactly 12582912 + 16d (|16d| < 2^22),
// and p = f32(scale/16) * (F - 12582912) = fma(scale/16, F,
// -(scale/16) * 12582912): the second product is exact (at most 13
// significant bits), so the fma rounds the exact product scale * d once, as
// f32(scale) * f32(d) does. Finite scales only: an infinite one gives NaN.
constexpr int kMagic = 0x4B400000;  // 12582912.0f
constexpr float kMagicF = 12582912.0f;

template <int JT, int LA>
__global__ __launch_bounds__(kDenseThreads) void w4a8_linear_dense_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq, int N, int K,
    int nwg, int Tr, const float* __restrict__ xs, float* __restrict__ y) {
    // slot sums of a tile: [buffer][slot][tt][i][q][row], token 16tt + 4q + i;
    // before the first tile, the activation staging buffers
    extern __shared__ __attribute__((aligned(16))) float red[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int s = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int G = K >> 5;
    const int NT = (N + 15) >> 4;
    const int b = blockIdx.x;
    const int ntiles = b < NT ? (NT - b + nwg - 1) / nwg : 0;
    if (ntiles == 0) return;

    const auto rw = make_rsrc(wq, (uint32_t)packed_weight_bytes(N, K));
    const auto rs = make_rsrc(wsg, (uint32_t)packed_scale_bytes(N, K));
    const auto rx = make_rsrc(xq, (uint32_t)(Tr * K));

    // Weights of iteration j of a tile: word q of row r's chunk of group
    // 16j + s, and its scale. The (tile, group) part of the offset is the
    // same for the whole wave and goes in the scalar offset; groups past G
    // and tiles past the list read through an empty resource, so they read
    // zeros. Offsets stay below 2^31.
    // LA tiles are in flight: buffer p holds the tiles k = p (mod LA).
    const auto rnull = make_rsrc(wq, 0u);
    const uint32_t lw = 16u * (uint32_t)r + 4u * (uint32_t)q, ls = 2u * (uint32_t)r;
    uint32_t w[LA][JT];
    uint16_t sc[LA][JT];
    auto wload = [&](int p, int j, int tile, bool past) {
        const int g = 16 * j + s;
        const bool bad = g >= G || past;
        const uint32_t chunk = (uint32_t)tile * (uint32_t)G + (uint32_t)g;
        w[p][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(bad ? rnull : rw, lw, bad ? 0u : chunk * 256u,
                                                                 kCachePolicyNT);
        sc[p][j] = __builtin_amdgcn_raw_buffer_load_b16(bad ? rnull : rs, ls, bad ? 0u : chunk * 32u,
                                                        kCachePolicyNT);
    };
    // the finishing thread's token scale: thread f < 512 finishes token
    // 16tt + 4q + i, row r of each tile, with (tt, i, q, r) = bits of f
    const int ftok = 16 * (tid >> 8) + 4 * ((tid >> 4) & 3) + ((tid >> 6) & 3);
    const float fxs = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(xs, (uint32_t)(4 * Tr)),
                                                    (4u * (uint32_t)ftok) | (tid < 512 ? 0u : kOOB), 0, 0));

    // A operands a[j][tt]: token 16tt + r, inputs 32(16j + s) + 8q .. +7.
    // The workgroup loads the activations coalesced (each token's
    // kStageGroups groups are 1 KB in a row), chunk by chunk, into LDS
    // (two alternating buffers); each wave then reads its own pieces. Tokens
    // past Tr and groups past G read zeros. Every chunk's loads go out
    // first, ahead of the weights: at the start of a launch all CUs ask for
    // their first tiles at once, and the shared activation rows would
    // otherwise queue behind them. The first tile's weights follow once the
    // first chunk is in, the second's after the staging.
    constexpr int NC = (16 * JT + kStageGroups - 1) / kStageGroups;  // chunks
    constexpr int RND = 32 * kStageGroups * 32 / 16 / kDenseThreads;  // 16-byte loads per thread and chunk
    v4i stage[NC][RND];
#pragma unroll
    for (int c = 0; c < NC; c++)
#pragma unroll
        for (int i = 0; i < RND; i++) {
            const int e = i * kDenseThreads + tid;
            const int t = e / (2 * kStageGroups), u = e % (2 * kStageGroups);
            const int g = c * kStageGroups + (u >> 1);
            const bool ok = t < Tr && g < G;
            stage[c][i] = load16(rx, ((uint32_t)(t * K + 32 * g + 16 * (u & 1))) | (ok ? 0u : kOOB));
        }
    long a[JT][2];
    char* lds = reinterpret_cast<char*>(red);
#pragma unroll
    for (int c = 0; c < NC; c++) {
        char* buf = lds + (c & 1) * kStageBytes;
#pragma unroll
        for (int i = 0; i < RND; i++) {
            const int e = i * kDenseThreads + tid;
            const int t = e / (2 * kStageGroups), u = e % (2 * kStageGroups);
            *reinterpret_cast<v4i*>(buf + ((u >> 1) * 33 + t) * 32 + 16 * (u & 1)) = stage[c][i];
        }
        // (a wave writes chunk c + 2 into this buffer only after every wave
        // has passed the next chunk's barrier, so after these reads)
        __syncthreads();
        if (c == 0) {
#pragma unroll
            for (int j = 0; j < JT; j++) wload(0, j, b, false);
        }
#pragma unroll
        for (int jj = 0; jj < kStageGroups / 16; jj++) {
            const int j = c * (kStageGroups / 16) + jj;  // group 16j + s = c * kStageGroups + 16jj + s
            if (j < JT) {
#pragma unroll
                for (int tt = 0; tt < 2; tt++) {
                    uint2 v = *reinterpret_cast<const uint2*>(buf + ((16 * jj + s) * 33 + 16 * tt + r) * 32 + 8 * q);
                    a[j][tt] = even_odd8((uint64_t)v.x | ((uint64_t)v.y << 32));
                }
            }
        }
    }
    __syncthreads();  // the staging area becomes the slot-sum buffers
#pragma unroll
    for (int p = 1; p < LA; p++)
#pragma unroll
        for (int j = 0; j < JT; j++) wload(p, j, b + p * nwg, p >= ntiles);
    // the token scale has arrived with the activations (taking it here keeps
    // the finish of every tile from waiting on the loads in flight)
    asm volatile("" ::"v"(fxs));
    const v4i bias = v4i{kMagic, kMagic, kMagic, kMagic};

    auto tile_body = [&](auto ptag, int k) {
        constexpr int p = decltype(ptag)::value;
        const int tile = b + k * nwg;
        const bool past = k + LA >= ntiles;
        float acc[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[tt][i] = 0.0f;
        // iteration j's products are issued before iteration j - 1's
        // scaling, so the matrix core works while the VALU scales
        v4i d[2][2];
        float s16[2];
        auto issue = [&](int j) {
            const long bw = decode_word(w[p][j]);
            s16[j & 1] = (float)__builtin_bit_cast(_Float16, sc[p][j]) * 0.0625f;
            d[j & 1][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[j][0], bw, bias, 0, 0, 0);
            d[j & 1][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[j][1], bw, bias, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            wload(p, j, tile + LA * nwg, past);  // iteration j of the tile LA ahead
            __builtin_amdgcn_sched_barrier(0);
        };
        auto scale = [&](int j) {
            const float m = s16[j & 1];
            const float c = -(m * kMagicF);
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int di = d[j & 1][tt][i];  // (a bit cast of the vector element itself reads element 0)
                    acc[tt][i] = acc[tt][i] + __builtin_fmaf(m, __builtin_bit_cast(float, di), c);
                }
        };
        issue(0);
#pragma unroll
        for (int j = 0; j < JT; j++) {
            if (j + 1 < JT) issue(j + 1);
            scale(j);
        }
        // the 16 slot sums of each (token, row): [slot][tt][i][q][r] in the
        // buffer of this tile's parity (a tile's reads of it end before any
        // thread passes the next tile's barrier)
        float* rb = red + (k & 1) * (16 * 512);
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) rb[s * 512 + ((tt * 4 + i) * 4 + q) * 16 + r] = acc[tt][i];
        __syncthreads();
        if (tid < 512) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) v[u] = rb[u * 512 + tid];
#pragma unroll
            for (int wd = 1; wd < 16; wd <<= 1)
#pragma unroll
                for (int u = 0; u < 16; u += 2 * wd) v[u] = v[u] + v[u + wd];
            const int row = 16 * tile + (tid & 15);
            if (ftok < Tr && row < N) y[(int64_t)ftok * N + row] = fxs * v[0];
        }
    };
    // groups of LA tiles, then the rest (no branch inside a group keeps the
    // load counts exact)
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    int k = 0;
    for (; k + LA <= ntiles; k += LA) {
        tile_body(I0{}, k);
        if constexpr (LA > 1) tile_body(I1{}, k + 1);
        if constexpr (LA > 2) tile_body(I2{}, k + 2);
        if constexpr (LA > 3) tile_body(I3{}, k + 3);
    }
    if constexpr (LA > 1)
        if (k < ntiles) tile_body(I0{}, k);
    if constexpr (LA > 2)
        if (k + 1 < ntiles) tile_body(I1{}, k + 1);
    if constexpr (LA > 3)
        if (k + 2 < ntiles) tile_body(I2{}, k + 2);
}

// Longer rows (kDenseMaxJ < J <= kDensePassMaxJ iterations per tile, e.g.
// the 14336-input down projection): the same dense products and order, but
// the activation operands do not fit in registers, so for every tile they
// stream through LDS in passes of one staging chunk (kStageGroups groups:
// iterations 2c and 2c + 1). A pass stores its chunk and issues the loads of
// the pass kDensePassAhead on: that chunk, and the weights of its two
// iterations into the registers just consumed (past the tile's end, those
// of the next tile), so every load has the same lead; then it issues both
// iterations' products before it scales them. Measured on MI355X (the 8B
// down projection, 32 tokens), the pass loop with no memory traffic at all
// takes 12.4 of the 21.0 us: the two fp32 operations per scaled group
// product (packed fp32 forms are not used) bound it, not the loads.
constexpr int kDensePassMaxJ = 28;
template <int JT>
__global__ __launch_bounds__(kDenseThreads) void w4a8_linear_dense_pass_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq, int N, int K,
    int nwg, int Tr, const float* __restrict__ xs, float* __restrict__ y) {
    constexpr int NP = JT / 2;              // passes per tile
    constexpr int SA = kDensePassAhead;     // passes whose loads are in flight
    constexpr int R = 2 * SA;               // weight iterations in flight: iteration j's registers take j + R next
    static_assert(JT % 2 == 0 && NP >= SA, "a pass takes two iterations");
    // two staging buffers, then two buffers of slot sums [slot][tt][i][q][row]
    extern __shared__ __attribute__((aligned(16))) float smem[];
    char* stg = reinterpret_cast<char*>(smem);
    float* red = reinterpret_cast<float*>(stg + 2 * kStageBytes);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int s = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int G = K >> 5;
    const int NT = (N + 15) >> 4;
    const int b = blockIdx.x;
    const int ntiles = b < NT ? (NT - b + nwg - 1) / nwg : 0;
    if (ntiles == 0) return;

    const auto rw = make_rsrc(wq, (uint32_t)packed_weight_bytes(N, K));
    const auto rs = make_rsrc(wsg, (uint32_t)packed_scale_bytes(N, K));
    const auto rx = make_rsrc(xq, (uint32_t)(Tr * K));
    // lane offsets, and the same with the out-of-range bit: groups past G and
    // tiles past the list read zeros through the range check
    const uint32_t lw = 16u * (uint32_t)r + 4u * (uint32_t)q, ls = 2u * (uint32_t)r;
    const uint32_t lwx = lw | kOOB, lsx = ls | kOOB;
    uint32_t w[R];
    uint16_t sc[R];
    auto wload = [&](int slot, int j, int tile, bool past) {  // iteration j of a tile, as in the kernel above
        const int g = 16 * j + s;
        const bool bad = g >= G || past;
        const uint32_t chunk = (uint32_t)tile * (uint32_t)G + (uint32_t)g;
        w[slot] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rw, bad ? lwx : lw, bad ? 0u : chunk * 256u,
                                                                 kCachePolicyNT);
        sc[slot] = __builtin_amdgcn_raw_buffer_load_b16(rs, bad ? lsx : ls, bad ? 0u : chunk * 32u, kCachePolicyNT);
    };
    // chunk c: groups 32c .. 32c + 31 of every token, 2 x 16 bytes per thread,
    // coalesced (each token's chunk is 1 KB in a row); tokens past Tr, groups
    // past G and chunks of no further tile read zeros
    constexpr int RND = 32 * kStageGroups * 32 / 16 / kDenseThreads;
    v4i stage[SA][RND];
    auto sload = [&](int sb, int c, bool none) {
#pragma unroll
        for (int i = 0; i < RND; i++) {
            const int e = i * kDenseThreads + tid;
            const int t = e / (2 * kStageGroups), u = e % (2 * kStageGroups);
            const int g = c * kStageGroups + (u >> 1);
            const bool ok = !none && t < Tr && g < G;
            stage[sb][i] = load16(rx, ((uint32_t)(t * K + 32 * g + 16 * (u & 1))) | (ok ? 0u : kOOB));
        }
    };
    auto sstore = [&](int sb, char* buf) {
#pragma unroll
        for (int i = 0; i < RND; i++) {
            const int e = i * kDenseThreads + tid;
            const int t = e / (2 * kStageGroups), u = e % (2 * kStageGroups);
            *reinterpret_cast<v4i*>(buf + ((u >> 1) * 33 + t) * 32 + 16 * (u & 1)) = stage[sb][i];
        }
    };
#pragma unroll
    for (int c = 0; c < SA; c++) sload(c, c, false);
#pragma unroll
    for (int j = 0; j < R; j++) wload(j, j, b, false);
    // the finishing thread's token scale (as in the register-resident kernel)
    const int ftok = 16 * (tid >> 8) + 4 * ((tid >> 4) & 3) + ((tid >> 6) & 3);
    const float fxs = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(xs, (uint32_t)(4 * Tr)),
                                                    (4u * (uint32_t)ftok) | (tid < 512 ? 0u : kOOB), 0, 0));
    const v4i bias = v4i{kMagic, kMagic, kMagic, kMagic};

    for (int k = 0; k < ntiles; k++) {
        const int tile = b + k * nwg;
        const bool past = k + 1 >= ntiles;
        float acc[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[tt][i] = 0.0f;
#pragma unroll
        for (int c = 0; c < NP; c++) {
            char* buf = stg + (c & 1) * kStageBytes;
            // (the last reads of this buffer, two passes ago, ended before
            // every wave passed the previous pass's barrier)
            sstore(c % SA, buf);
            if (c + SA < NP)
                sload(c % SA, c + SA, false);
            else  // the next tile's first chunks: the same activation rows
                sload(c % SA, c + SA - NP, past);
            __syncthreads();
            v4i d[2][2];
            float s16[2];
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const int j = 2 * c + jj;  // group 16j + s = c * kStageGroups + 16jj + s
                long a[2];
#pragma unroll
                for (int tt = 0; tt < 2; tt++) {
                    const uint2 v = *reinterpret_cast<const uint2*>(buf + ((16 * jj + s) * 33 + 16 * tt + r) * 32 + 8 * q);
                    a[tt] = even_odd8((uint64_t)v.x | ((uint64_t)v.y << 32));
                }
                const long bw = decode_word(w[j % R]);
                s16[jj] = (float)__builtin_bit_cast(_Float16, sc[j % R]) * 0.0625f;
                d[jj][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[0], bw, bias, 0, 0, 0);
                d[jj][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[1], bw, bias, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (j + R < JT)  // iteration j + R of this tile, or j + R - JT of the next
                    wload(j % R, j + R, tile, false);
                else
                    wload(j % R, j + R - JT, tile + nwg, past);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const float m = s16[jj];
                const float cb = -(m * kMagicF);
#pragma unroll
                for (int tt = 0; tt < 2; tt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int di = d[jj][tt][i];
                        acc[tt][i] = acc[tt][i] + __builtin_fmaf(m, __builtin_bit_cast(float, di), cb);
                    }
            }
        }
        // the 16 slot sums of each (token, row), added as the index-order tree
        float* rb = red + (k & 1) * (16 * 512);
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) rb[s * 512 + ((tt * 4 + i) * 4 + q) * 16 + r] = acc[tt][i];
        __syncthreads();
        if (tid < 512) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) v[u] = rb[u * 512 + tid];
#pragma unroll
            for (int wd = 1; wd < 16; wd <<= 1)
#pragma unroll
                for (int u = 0; u < 16; u += 2 * wd) v[u] = v[u] + v[u + wd];
            const int row = 16 * tile + (tid & 15);
            if (ftok < Tr && row < N) y[(int64_t)ftok * N + row] = fxs * v[0];
        }
    }
}

constexpr size_t kDensePassLds = (size_t)2 * kStageBytes + (size_t)2 * 16 * 512 * sizeof(float);

// Dynamic LDS: the two activation staging buffers, later two buffers of 16
// slots x 512 (token, row) sums.
constexpr size_t kDenseLds = (size_t)2 * kStageBytes > (size_t)2 * 16 * 512 * sizeof(float)
                                 ? (size_t)2 * kStageBytes
                                 : (size_t)2 * 16 * 512 * sizeof(float);

static int dense_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int JT>
static int launch_dense(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, int Tr,
                        int N, int K, hipStream_t s) {
    // two tiles in flight where the registers allow it
    auto kernel = &w4a8_linear_dense_kernel<JT, JT <= 8 ? kDenseLookahead : 1>;
    static bool enabled = false;
    if (!enabled) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)kDenseLds) != hipSuccess) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        enabled = true;
    }
    const int NT = (N + 15) / 16;
    const int cus = dense_cus();
    const int grid = NT < cus ? NT : cus;  // one workgroup of 16 waves per CU
    hipEvent_t e0, e1;
    if (take_linear_timing(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kDenseThreads), kDenseLds, s, e0, e1, 0, wq, ws, xq, N, K,
                              grid, Tr, xs, y);
    else
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kDenseThreads), kDenseLds, s, wq, ws, xq, N, K, grid, Tr, xs, y);
    return launch_status();
}

template <int JT>
static int launch_dense_pass(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                             int Tr, int N, int K, hipStream_t s) {
    auto kernel = &w4a8_linear_dense_pass_kernel<JT>;
    static bool enabled = false;
    if (!enabled) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)kDensePassLds) != hipSuccess) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        enabled = true;
    }
    const int NT = (N + 15) / 16;
    const int cus = dense_cus();
    const int grid = NT < cus ? NT : cus;
    hipEvent_t e0, e1;
    if (take_linear_timing(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kDenseThreads), kDensePassLds, s, e0, e1, 0, wq, ws, xq, N, K,
                              grid, Tr, xs, y);
    else
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kDenseThreads), kDensePassLds, s, wq, ws, xq, N, K, grid, Tr, xs,
                           y);
    return launch_status();
}

bool linear_dense_supported(int T, int K) {
    const int J = (K / 32 + 15) / 16;
    return T > 16 && T <= kDenseTokens && K >= 32 && K % 32 == 0 && J <= kDensePassMaxJ;
}

// Iterations per tile rounded up to a compiled count (extra iterations read
// zeros and add +0, which leaves a slot unchanged).
int linear_dense_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, int T,
                         int N, int K, hipStream_t s) {
    if (!linear_dense_supported(T, K)) return SPECV_E_SHAPE;
    const int J = (K / 32 + 15) / 16;
    // Workgroups of at most two tiles stream their activation operands too:
    // staging all of them into registers up front costs more than a tile or
    // two use (measured on MI355X at 32 tokens, K = 4096, per launch: qkv
    // 11.8 -> 10.9 us, o 7.86 -> 7.35 us; with gate_up's 7 tiles per
    // workgroup 27 -> 35 us, so longer walks keep the registers).
    const int NT = (N + 15) / 16;
    if (J > 4 && J <= kDenseMaxJ && NT <= 2 * dense_cus())
        return J <= 8 ? launch_dense_pass<8>(wq, ws, xq, xs, y, T, N, K, s)
                      : launch_dense_pass<10>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= 1) return launch_dense<1>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= 2) return launch_dense<2>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= 4) return launch_dense<4>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= 8) return launch_dense<8>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= kDenseMaxJ) return launch_dense<10>(wq, ws, xq, xs, y, T, N, K, s);
    if (J <= 16) return launch_dense_pass<16>(wq, ws, xq, xs, y, T, N, K, s);
    return launch_dense_pass<kDensePassMaxJ>(wq, ws, xq, xs, y, T, N, K, s);
}

}  // namespace specv
