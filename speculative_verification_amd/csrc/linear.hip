// W4A8 linear for T = 1..16 tokens on CDNA4 matrix cores.
//
// Operation (GPU-Resident Speculative Decoding for In-Browser LLM Inference
// with WebGPU, Small-Batch Verification Kernels and Implementation):
//   d[t][n][g] = sum_{k in group g} q(n,k) * xq[t][k]   exact int32
//   p_g        = f32(scale[g][n]) * f32(d)               one rounding
//   y[t][n]    = xs[t] * R16(p_0 .. p_{G-1})             fixed order
// R16: slot s in 0..15 accumulates the groups g = s, s+16, s+32, ... in
// increasing g from +0; the 16 slots are then added as a binary tree in
// index order (slot s += slot s+w for s divisible by 2w, w = 1, 2, 4, 8).
// An iteration j covers the 16 groups 16j .. 16j+15, one per slot; the 16
// slots form four quads of four.
//
// Work decomposition, two layouts chosen per shape:
//  stream: the default. About two workgroups per CU, each walking a list of
//          16-row tiles; its four waves take the four slot quads of every
//          tile (wave w: groups 16j + 4w + 0..3, 64 contiguous bytes per row
//          per iteration). A wave keeps its quarter of the activation codes
//          in LDS after loading it with its first tile, and its weight loads
//          run a fixed number of iterations ahead, across tile boundaries.
//  split:  for shapes whose activations do not fit in LDS (T x K large): 64
//          rows and one of S = 2 or 4 K-slices per workgroup; each slice
//          reduces its own slots and the last workgroup of a row group to
//          finish adds the S partials in tree order.
//
// Integer dots. One v_mfma_i32_16x16x64_i8 computes, for 16 rows, the dots
// of 16 inputs of each group of a slot quad against up to four tokens: B
// (64x16) carries the weights, lane quarter q supplying 16 inputs of slot q
// of the quad for row l%16; A (16x64) carries the activations
// block-diagonally, row m = 4h+t holding token t's same 16 inputs of slot h
// in k-quarter h and zeros elsewhere. A and B share one lane layout, so byte
// b of an A lane meets byte b of the B lane of the same quarter, and output
// element (m, n) = (4h+t, row) is exactly the 16-input dot of row n, slot h,
// token t; it lands in lane 16h + n, register t: the lane that loaded that
// row's group and scale. Two such products accumulate in the int32
// accumulator, giving the exact group dot.
//
// Nibble decode. Codes are stored u = q + 8. Flipping bit 3 of each nibble
// gives the 4-bit two's complement of q; moving it into the high half of a
// byte gives the int8 value 16q: the even inputs of a word come out of its
// low nibbles, the odd inputs out of its high nibbles, with no byte permute,
// because the staged activations of each 8-input chunk are stored in the same
// even-then-odd order. The dots therefore come out as 16d (exact,
// |16d| < 2^20), and the scale is pre-divided by 16 (exact: a power of two on
// a widened fp16 value), so f32(scale/16) * f32(16d) is the same real product
// as f32(scale) * f32(d) and rounds identically.
//
// Ragged shapes. All global loads go through buffer resources, whose range
// check returns zeros. Rows past N lie past the end of the weights; groups
// past G read zeros (an out-of-range offset) against zero activations, so
// they add +0, which never changes a slot (a slot is never -0).
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"

namespace specv {

// Weight iterations in flight per wave, and streaming workgroups per CU.
#ifndef SPECV_STREAM_STAGES
#define SPECV_STREAM_STAGES 4
#endif
#ifndef SPECV_STREAM_WGS_PER_CU
#define SPECV_STREAM_WGS_PER_CU 2
#endif
#ifndef SPECV_SPLIT_STAGES
#define SPECV_SPLIT_STAGES 2
#endif

// Integer dots of one group per slot of a quad (see the header): w is the
// lane's 16 bytes of nibbles (32 inputs of its slot's group, row l%16); a0
// and a1 are the lane's A operands for inputs 0..15 and 16..31 of each token
// tile of 4. d[tt] receives 16 x the exact group dots.
template <int TT>
__device__ __forceinline__ void quad_dots(const v4i w, const v4i (&a0)[TT], const v4i (&a1)[TT], v4i (&d)[TT]) {
    v4i b[2];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const unsigned W = (unsigned)w[c];
        b[c >> 1][2 * (c & 1)] = (int)(((W << 4) ^ 0x80808080u) & 0xF0F0F0F0u);  // inputs 0, 2, 4, 6
        b[c >> 1][2 * (c & 1) + 1] = (int)((W ^ 0x80808080u) & 0xF0F0F0F0u);     // inputs 1, 3, 5, 7
    }
#pragma unroll
    for (int tt = 0; tt < TT; tt++) d[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[tt], b[0], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
    for (int tt = 0; tt < TT; tt++) d[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[tt], b[1], d[tt], 0, 0, 0);
}

// Activation codes of one 16-byte chunk (two 8-input chunks) in the
// even-then-odd order of the nibble decode: inputs 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ v4i even_odd(const v4i a) {
    return v4i{(int)__builtin_amdgcn_perm(a[1], a[0], 0x06040200u), (int)__builtin_amdgcn_perm(a[1], a[0], 0x07050301u),
               (int)__builtin_amdgcn_perm(a[3], a[2], 0x06040200u), (int)__builtin_amdgcn_perm(a[3], a[2], 0x07050301u)};
}

// ---------------------------------------------------------------- stream

// Streaming layout. The grid is a multiple of 32 workgroups; workgroup b
// walks the 16-row tiles v, v + nwg, v + 2 nwg, ... Its four waves take the
// four slot quads of every tile, so a wave only ever uses its own quarter of
// each token's activation codes: it loads that quarter together with the
// first tile's weights, iteration by iteration, stores it in LDS in the MFMA
// operand order, and reads it back from there for every later tile (the
// activations cross the CU once per workgroup instead of once per 16 rows).
// Slot pp of the load pipeline holds iterations pp, pp + P, ... of a tile,
// and in the tile's last block it is refilled with iteration pp of the next
// tile, so the stream does not drain between tiles. At the end of a tile the
// four quad sums of each row meet in LDS (tree levels w = 4, 8) and 16T
// threads scale and store them. With an argmax, each of those threads keeps
// the best of its rows over the tiles, and the workgroup writes one (value,
// lowest row) pair per token.
constexpr int kStreamZero = 64;  // zero bytes after the staged activations

template <int T>
struct SStage {
    v4i w;              // 16 bytes of nibbles: one group of one row
    uint16_t s;         // its fp16 scale
    v4i x[(T + 7) / 8]; // first tile only: 16 bytes of this wave's activation quarter per 8 tokens
};

// The arguments the first loads need come first: with kernel-argument
// preloading the first 14 dwords arrive in SGPRs, and the rest (the argmax
// output, used last) is fetched while the stream starts.
template <int T, int P, bool AMAX>
__global__ __launch_bounds__(256) void w4a8_linear_stream_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq, int N, int K,
    int nwg, const float* __restrict__ xs, float* __restrict__ y, int write_y, Best* __restrict__ amax) {
    constexpr int TT = (T + 3) / 4;
    constexpr int TX = (T + 7) / 8;
    extern __shared__ __attribute__((aligned(16))) int8_t act[];
    __shared__ float red[2][4][T][16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;         // row within the tile; MFMA column n
    const int q = lane >> 4;         // slot within the quad; k-quarter of B
    const int h = (lane & 15) >> 2;  // slot of this lane's A row
    const int tp = lane & 3;         // token of this lane's A row within a tile of 4
    const int G = K >> 5;
    const int J = (G + 15) >> 4;
    const int JP = (J + P - 1) / P * P;  // iterations per tile, padded to whole blocks of P
    const int NT = (N + 15) >> 4;
    // The four 16-row tiles of a 64-row block share the 128-byte lines of
    // their group-major scales: they go to workgroups that the hardware's
    // round-robin placement (workgroup b on XCD b mod 8) puts on one XCD,
    // whose L2 then fetches each line once. nwg being a multiple of 32 keeps
    // that true for every tile of the lists.
    const int b = blockIdx.x, ib = b >> 3;
    const int v = 4 * ((ib >> 2) * 8 + (b & 7)) + (ib & 3);
    const int ntiles = v < NT ? (NT - v + nwg - 1) / nwg : 0;

    // finishing thread of a tile: token ft, row fr
    const int ft = tid >> 4, fr = tid & 15;
    const bool fin = tid < 16 * T;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    if (ntiles == 0) {
        if (AMAX && fin && fr == 0) amax[(int64_t)ft * nwg + b] = Best{bv, bi};
        return;
    }
    const float fxs = fin ? xs[ft] : 0.0f;

    const auto rw = make_rsrc(wq, (uint32_t)((int64_t)N * (K / 2)));
    const auto rs = make_rsrc(wsg, (uint32_t)((int64_t)G * N * 2));
    const auto rx = make_rsrc(xq, (uint32_t)(T * K));
    const uint32_t lq = 4u * wave + q;  // group of this lane within an iteration
    const int xc = lane & 7;            // 16-byte chunk of the quarter this lane loads
    const uint32_t xlane = 32u * (4u * wave + (xc >> 1)) + 16u * (xc & 1);

    // One iteration j of a tile: the lane's 16 bytes of nibbles and scale, and
    // on the first tile 16 bytes of activation codes per 8 tokens. Every load
    // is issued unconditionally, so the compiler counts them statically: a
    // row past N lies past the weights, a group past G (a ragged or padding
    // iteration) and a tile past the list take the out-of-range bit, and all
    // of these read zeros. Offsets stay below 2^32: the weights and scales are
    // each under 2^31 bytes.
    auto load = [&](SStage<T>& st, int tile, int j, bool with_act, uint32_t past) {
        const uint32_t bad = ((16 * j + (int)lq >= G) ? kOOB : 0u) | past;
        const uint32_t row = 16u * (uint32_t)tile + (uint32_t)r;
        st.w = load16(rw, (row * (uint32_t)(K / 2) + 16u * lq + 256u * (uint32_t)j) | bad);
        st.s = load2(rs, ((((uint32_t)(16 * j) + lq) * (uint32_t)N + row) * 2u) | bad);
        if (with_act) {
#pragma unroll
            for (int x = 0; x < TX; x++) {
                const int xt = (lane >> 3) + 8 * x;
                const bool ok = xt < T && 16 * j + 4 * wave + (xc >> 1) < G;
                st.x[x] = load16(rx, ((uint32_t)(xt * K + 512 * j) + xlane) | (ok ? 0u : kOOB));
            }
        }
    };
    // Activation chunks go to LDS as [t][j][wave][128 bytes] (padding
    // iterations store zeros). Only this wave reads its quarter, and a wave's
    // LDS accesses complete in order, so no barrier is needed.
    auto put_act = [&](const SStage<T>& st, int j) {
#pragma unroll
        for (int x = 0; x < TX; x++) {
            const int xt = (lane >> 3) + 8 * x;
            if (xt < T) *reinterpret_cast<v4i*>(act + ((xt * JP + j) * 4 + wave) * 128 + 16 * xc) = even_odd(st.x[x]);
        }
    };

    // A operand addresses: token t = 4tt + tp of slot h, advanced by one
    // iteration per j; lanes whose A row is zero stay on the zero bytes.
    const int zero_off = T * JP * 512;
    int abase[TT], astep[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int t = 4 * tt + tp;
        const bool ok = q == h && t < T;
        abase[tt] = ok ? (t * JP * 4 + wave) * 128 + h * 32 : zero_off;
        astep[tt] = ok ? 512 : 0;
    }
    auto compute = [&](const SStage<T>& st, int j, float (&acc)[T]) {
        v4i a0[TT], a1[TT], d[TT];
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            const int off = abase[tt] + j * astep[tt];
            a0[tt] = *reinterpret_cast<const v4i*>(act + off);
            a1[tt] = *reinterpret_cast<const v4i*>(act + off + 16);
        }
        quad_dots<TT>(st.w, a0, a1, d);
        const float s16 = (float)__builtin_bit_cast(_Float16, st.s) * 0.0625f;
#pragma unroll
        for (int tt = 0; tt < TT; tt++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (4 * tt + u < T) acc[4 * tt + u] = acc[4 * tt + u] + s16 * (float)d[tt][u];
    };

    SStage<T> st[P];
#pragma unroll
    for (int pp = 0; pp < P; pp++) {
        load(st[pp], v, pp, true, 0u);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < kStreamZero / 16) *reinterpret_cast<v4i*>(act + zero_off + 16 * tid) = v4i{0, 0, 0, 0};
    __syncthreads();

    auto run_tile = [&](auto first_tag, int k, float (&acc)[T]) {
        constexpr bool FIRST = decltype(first_tag)::value;
        const int tile = v + k * nwg;
        int j0 = 0;
        for (; j0 + P < JP; j0 += P) {
#pragma unroll
            for (int pp = 0; pp < P; pp++) {
                if (FIRST) put_act(st[pp], j0 + pp);
                compute(st[pp], j0 + pp, acc);
                __builtin_amdgcn_sched_barrier(0);
                load(st[pp], tile, j0 + pp + P, FIRST, 0u);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const uint32_t past = k + 1 < ntiles ? 0u : kOOB;
#pragma unroll
        for (int pp = 0; pp < P; pp++) {
            if (FIRST) put_act(st[pp], j0 + pp);
            compute(st[pp], j0 + pp, acc);
            __builtin_amdgcn_sched_barrier(0);
            load(st[pp], tile + nwg, pp, false, past);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // End of a tile: levels w = 1, 2 pair the four slots of a quad (lanes
    // q ^ 1, q ^ 2), levels w = 4, 8 the four waves' quads, in LDS. The
    // reduction buffer alternates between tiles: a tile's reads of it end
    // before any thread passes the next tile's barrier.
    auto finish_tile = [&](int k, const float (&acc)[T], int buf) {
        const int tile = v + k * nwg;
#pragma unroll
        for (int t = 0; t < T; t++) {
            float s = acc[t];
            s = s + __shfl_xor(s, 16, 64);
            s = s + __shfl_xor(s, 32, 64);
            if (q == 0) red[buf][wave][t][r] = s;
        }
        __syncthreads();
        if (fin) {
            const int row = 16 * tile + fr;
            const float val = fxs * ((red[buf][0][ft][fr] + red[buf][1][ft][fr]) +
                                     (red[buf][2][ft][fr] + red[buf][3][ft][fr]));
            if (row < N) {
                if (!AMAX || write_y) y[(int64_t)ft * N + row] = val;
                if (AMAX && better(val, row, bv, bi)) {
                    bv = val;
                    bi = row;
                }
            }
        }
    };
    {
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; t++) acc[t] = 0.0f;
        run_tile(std::true_type{}, 0, acc);
        finish_tile(0, acc, 0);
    }
    for (int k = 1; k < ntiles; k++) {
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; t++) acc[t] = 0.0f;
        run_tile(std::false_type{}, k, acc);
        finish_tile(k, acc, k & 1);
    }
    if (AMAX && fin) {
        best16(bv, bi);
        if (fr == 0) amax[(int64_t)ft * nwg + b] = Best{bv, bi};
    }
}

// ---------------------------------------------------------------- split

// Split-K layout: a workgroup owns 64 rows (4 waves x 16) and one of S
// K-slices, the Q = 4/S slot quads pQ .. pQ+Q-1 of every iteration. The S
// workgroups of a row group are numbered so that the round-robin placement
// puts them on one XCD, whose L2 serves the lines they share. A workgroup
// stages its slice's activations in LDS as [t][j][Q*128 bytes] (j below J
// rounded up to whole blocks of P, zeros past the last group), followed by
// kSplitZero zero bytes that lanes whose A operand must be zero read.
constexpr int kSplitZero = 512;

template <int Q>
struct WStage {
    v4i w[Q];       // per slot quad: 16 bytes of nibbles (one group of one row)
    uint16_t s[Q];  // and its fp16 scale
};

template <int T, int S>
__global__ __launch_bounds__(256) void w4a8_linear_split_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq,
    const float* __restrict__ xs, float* __restrict__ y, float* __restrict__ part, int* __restrict__ cnt, int N,
    int K) {
    constexpr int Q = 4 / S;  // slot quads of the slice
    constexpr int ROWS = 64;
    constexpr int TT = (T + 3) / 4;
    constexpr int P = SPECV_SPLIT_STAGES;
    extern __shared__ __attribute__((aligned(16))) int8_t act[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;
    const int q = lane >> 4;
    const int h = (lane & 15) >> 2;
    const int tp = lane & 3;
    const int G = K >> 5;
    const int J = (G + 15) >> 4;
    const int JP = (J + P - 1) / P * P;
    const int NG = (N + ROWS - 1) / ROWS;

    const int b = blockIdx.x, ib = b >> 3;
    const int p = ib % S;
    const int rg = (ib / S) * 8 + (b & 7);
    if (rg >= NG) return;
    const int row = rg * ROWS + wave * 16 + r;
    const bool row_ok = row < N;
    const int quad0 = p * Q;

    const auto rw = make_rsrc(wq, (uint32_t)((int64_t)N * (K / 2)));
    const auto rs = make_rsrc(wsg, (uint32_t)((int64_t)G * N * 2));
    const auto rx = make_rsrc(xq, (uint32_t)(T * K));

    // The steady loop's loads are plain (in range, not a ragged last
    // iteration); the last block or two take checked loads, where iterations
    // past J, and in a ragged last iteration the lanes past G, take the
    // out-of-range bit and read zeros.
    const uint32_t wlane = (uint32_t)row * (uint32_t)(K / 2) + 16u * (uint32_t)(4 * quad0 + q);
    const uint32_t slane = ((uint32_t)(4 * quad0 + q) * (uint32_t)N + (uint32_t)row) * 2u;
    const bool ragged = (G & 15) != 0;
    auto load_fast = [&](WStage<Q>& st, int j) {
        const uint32_t wo = wlane + 256u * (uint32_t)j;
        const uint32_t so = slane + 32u * (uint32_t)N * (uint32_t)j;
#pragma unroll
        for (int qq = 0; qq < Q; qq++) {
            st.w[qq] = load16(rw, wo + 64u * (uint32_t)qq);
            st.s[qq] = load2(rs, so + 8u * (uint32_t)N * (uint32_t)qq);
        }
    };
    auto load_stage = [&](WStage<Q>& st, int j) {
        const uint32_t wo = wlane + 256u * (uint32_t)j;
        const uint32_t so = slane + 32u * (uint32_t)N * (uint32_t)j;
        const uint32_t past = j >= J ? kOOB : 0u;
#pragma unroll
        for (int qq = 0; qq < Q; qq++) {
            const uint32_t bad = past | ((uint32_t)(16 * j + 4 * (quad0 + qq) + q >= G) << 31);
            st.w[qq] = load16(rw, (wo + 64u * (uint32_t)qq) | bad);
            st.s[qq] = load2(rs, (so + 8u * (uint32_t)N * (uint32_t)qq) | bad);
        }
    };

    WStage<Q> st[P];
#pragma unroll
    for (int pp = 0; pp < P; pp++) {
        load_stage(st[pp], pp);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Stage the slice's activations in rounds of U chunks per thread; the
    // loads of round r + 1 are issued before the LDS writes of round r, so
    // the rounds' L2 round trips overlap.
    const int nchunks = T * JP * Q * 8;  // 16-byte chunks
    constexpr int U = 8;
    auto stage_load = [&](v4i (&vv)[U], int base) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (base + u * 256 >= nchunks) break;
            const int i = base + u * 256 + tid;
            const int c = i % (Q * 8);
            const int tj = i / (Q * 8);
            const int j = tj % JP;
            const int t = tj / JP;
            const int g = 16 * j + 4 * quad0 + (c >> 1);
            const bool ok = i < nchunks && g < G;
            vv[u] = load16(rx, ((uint32_t)(t * K + 32 * g + 16 * (c & 1))) | ((uint32_t)!ok << 31));
        }
    };
    auto stage_store = [&](const v4i (&vv)[U], int base) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (base + u * 256 >= nchunks) break;
            const int i = base + u * 256 + tid;
            if (i < nchunks) *reinterpret_cast<v4i*>(act + 16 * i) = even_odd(vv[u]);
        }
    };
    {
        v4i va[U], vb[U];
        stage_load(va, 0);
        for (int base = 0; base < nchunks; base += 512 * U) {
            const bool more = base + 256 * U < nchunks;
            if (more) stage_load(vb, base + 256 * U);
            stage_store(va, base);
            if (!more) break;
            if (base + 512 * U < nchunks) stage_load(va, base + 512 * U);
            stage_store(vb, base + 256 * U);
        }
    }
    const int zero_off = nchunks * 16;
    if (tid < kSplitZero / 16) *reinterpret_cast<v4i*>(act + zero_off + 16 * tid) = v4i{0, 0, 0, 0};
    __syncthreads();

    float acc[Q][T];
#pragma unroll
    for (int qq = 0; qq < Q; qq++)
#pragma unroll
        for (int t = 0; t < T; t++) acc[qq][t] = 0.0f;

    int abase[TT], astep[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int t = 4 * tt + tp;
        const bool ok = q == h && t < T;
        abase[tt] = ok ? (t * JP * Q) * 128 + h * 32 : zero_off;
        astep[tt] = ok ? Q * 128 : 0;
    }
    auto compute = [&](const WStage<Q>& stg, int j) {
#pragma unroll
        for (int qq = 0; qq < Q; qq++) {
            v4i a0[TT], a1[TT], d[TT];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                const int off = abase[tt] + j * astep[tt] + qq * 128;  // zero lanes: within the zero bytes
                a0[tt] = *reinterpret_cast<const v4i*>(act + off);
                a1[tt] = *reinterpret_cast<const v4i*>(act + off + 16);
            }
            quad_dots<TT>(stg.w[qq], a0, a1, d);
            const float s16 = (float)__builtin_bit_cast(_Float16, stg.s[qq]) * 0.0625f;
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (4 * tt + u < T) acc[qq][4 * tt + u] = acc[qq][4 * tt + u] + s16 * (float)d[tt][u];
        }
    };

    const int Jsafe = ragged ? J - 1 : J;
    int j0 = 0;
    for (; j0 + 2 * P <= Jsafe; j0 += P) {
#pragma unroll
        for (int pp = 0; pp < P; pp++) {
            compute(st[pp], j0 + pp);
            __builtin_amdgcn_sched_barrier(0);
            load_fast(st[pp], j0 + pp + P);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    for (; j0 < J; j0 += P) {
#pragma unroll
        for (int pp = 0; pp < P; pp++) {
            compute(st[pp], j0 + pp);
            __builtin_amdgcn_sched_barrier(0);
            load_stage(st[pp], j0 + pp + P);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Tree levels w = 1, 2 pair the four slots of a quad (lanes q ^ 1, q ^ 2);
    // with two quads, level w = 4 adds them inside the lane.
    float val[Q][T];
#pragma unroll
    for (int qq = 0; qq < Q; qq++)
#pragma unroll
        for (int t = 0; t < T; t++) {
            float v = acc[qq][t];
            v = v + __shfl_xor(v, 16, 64);
            v = v + __shfl_xor(v, 32, 64);
            val[qq][t] = v;
        }

    // Partials and counters use device-scope relaxed atomic accesses: they
    // are coherent across the XCDs' separate L2 caches without a device-scope
    // fence (which would write back the whole L2). All partial stores of the
    // workgroup complete (s_waitcnt, then the barrier) before its counter
    // increment, so the workgroup that observes the final count reads every
    // partial.
    if (q == 0 && row_ok)
#pragma unroll
        for (int t = 0; t < T; t++)
            __hip_atomic_store(&part[((int64_t)p * T + t) * N + row], (Q == 2) ? (val[0][t] + val[1 % Q][t]) : val[0][t],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        s_last = (__hip_atomic_fetch_add(&cnt[rg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1);
    __syncthreads();
    if (!s_last) return;
    const int64_t ps = (int64_t)T * N;
    for (int idx = tid; idx < ROWS * T; idx += 256) {
        const int t = idx / ROWS;
        const int orow = rg * ROWS + idx % ROWS;
        if (orow >= N) continue;
        float* pp = part + (int64_t)t * N + orow;
        float v[S];
#pragma unroll
        for (int k = 0; k < S; k++) v[k] = __hip_atomic_load(pp + k * ps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float tot = (S == 2) ? v[0] + v[1 % S] : (v[0] + v[1 % S]) + (v[2 % S] + v[3 % S]);
        y[(int64_t)t * N + orow] = xs[t] * tot;
    }
    if (tid == 0) __hip_atomic_store(&cnt[rg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- host

constexpr size_t kLdsBudget = 150 * 1024;
enum { kStream = 1 };  // layout; a split layout is its slice count S in {2, 4}

// Dynamic LDS of a streaming workgroup (its tile reduction buffer, 512T
// bytes, is static).
inline size_t stream_lds_bytes(int T, int K) {
    const int J = (K / 32 + 15) / 16;
    const int JP = (J + SPECV_STREAM_STAGES - 1) / SPECV_STREAM_STAGES * SPECV_STREAM_STAGES;
    return (size_t)T * JP * 512 + kStreamZero;
}
inline bool stream_fits(int T, int K) { return stream_lds_bytes(T, K) + (size_t)T * 512 <= kLdsBudget; }

// Staged activation bytes of a split workgroup with S slices.
inline size_t split_lds_bytes(int T, int K, int S) {
    const int J = (K / 32 + 15) / 16;
    const int JP = (J + SPECV_SPLIT_STAGES - 1) / SPECV_SPLIT_STAGES * SPECV_SPLIT_STAGES;
    return (size_t)T * JP * (4 / S) * 128 + kSplitZero;
}

// Compute units of the current device (cached per device).
static int device_cus() {
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

// Workgroups of a streaming launch: a multiple of 32 (the tile numbering
// needs it), no more than the tiles need, about WGS_PER_CU per CU.
inline int stream_grid(int N) {
    const int NT = (N + 15) / 16;
    const int cap = (device_cus() * SPECV_STREAM_WGS_PER_CU + 31) / 32 * 32;
    const int need = (NT + 31) / 32 * 32;
    return need < cap ? need : cap;
}

// Layout for a shape: streaming when a wave's activation quarter of every
// token fits in LDS; otherwise K split in 2 slices (many rows) or 4.
inline int linear_mode(int T, int N, int K) {
    if (stream_fits(T, K)) return kStream;
    return split_lds_bytes(T, K, 2) <= kLdsBudget && (N + 63) / 64 >= 256 ? 2 : 4;
}

inline int linear_row_groups_padded(int N) {
    const int NG = (N + 63) / 64;
    return (NG + 7) / 8 * 8;
}

// Split-K workspace: one counter per row group in a fixed region sized for
// the largest N (so its location never depends on the call), then the
// partials. Only the counters must start at zero; every call returns the
// counters it used to zero, and partials are written before they are read.
constexpr size_t kCounterBytes = (size_t)((1 << 24) / 64) * 4;

// Events for the next linear launch of this host thread (timing diagnostics).
static thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;

// Dynamic LDS above 64 KB must be enabled per kernel, up to what the launch
// needs (the static LDS of the kernel counts towards the limit).
static int enable_lds(const void* kernel, size_t lds, size_t& enabled) {
    if (lds <= enabled) return SPECV_OK;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
        (void)hipGetLastError();
        return SPECV_E_HIP;
    }
    enabled = lds;
    return SPECV_OK;
}

template <int T>
static int launch_stream(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                         Best* amax, int N, int K, hipStream_t s) {
    constexpr int P = SPECV_STREAM_STAGES;
    const int write_y = y != nullptr;
    static size_t lds_enabled = 64 * 1024;
    const size_t lds = stream_lds_bytes(T, K);
    if (!stream_fits(T, K)) return SPECV_E_SHAPE;
    const int grid = stream_grid(N);
    auto go = [&](auto kernel, size_t& enabled) {
        const int rc = enable_lds(reinterpret_cast<const void*>(kernel), lds, enabled);
        if (rc != SPECV_OK) return rc;
        if (g_time_start) {
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), lds, s, g_time_start, g_time_stop, 0, wq, ws, xq, N,
                                  K, grid, xs, y, write_y, amax);
            g_time_start = g_time_stop = nullptr;
        } else {
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), lds, s, wq, ws, xq, N, K, grid, xs, y, write_y, amax);
        }
        return launch_status();
    };
    static size_t lds_enabled_amax = 64 * 1024;
    return amax ? go(&w4a8_linear_stream_kernel<T, P, true>, lds_enabled_amax)
                : go(&w4a8_linear_stream_kernel<T, P, false>, lds_enabled);
}

template <int T, int S>
static int launch_split(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                        float* part, int* cnt, int N, int K, hipStream_t s) {
    static size_t lds_enabled = 64 * 1024;
    const size_t lds = split_lds_bytes(T, K, S);
    if (lds > kLdsBudget) return SPECV_E_SHAPE;
    const int rc = enable_lds(reinterpret_cast<const void*>(&w4a8_linear_split_kernel<T, S>), lds, lds_enabled);
    if (rc != SPECV_OK) return rc;
    const int grid = S * linear_row_groups_padded(N);
    if (g_time_start) {
        hipExtLaunchKernelGGL((w4a8_linear_split_kernel<T, S>), dim3(grid), dim3(256), lds, s, g_time_start,
                              g_time_stop, 0, wq, ws, xq, xs, y, part, cnt, N, K);
        g_time_start = g_time_stop = nullptr;
    } else {
        hipLaunchKernelGGL((w4a8_linear_split_kernel<T, S>), dim3(grid), dim3(256), lds, s, wq, ws, xq, xs, y, part,
                           cnt, N, K);
    }
    return launch_status();
}

template <int T>
static int launch_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                    Best* amax, float* part, int* cnt, int N, int K, hipStream_t s) {
    switch (linear_mode(T, N, K)) {
        case kStream: return launch_stream<T>(wq, ws, xq, xs, y, amax, N, K, s);
        case 2: return amax ? SPECV_E_SHAPE : launch_split<T, 2>(wq, ws, xq, xs, y, part, cnt, N, K, s);
        default: return amax ? SPECV_E_SHAPE : launch_split<T, 4>(wq, ws, xq, xs, y, part, cnt, N, K, s);
    }
}

// Finishes the argmax of each token from its workgroups' (value, row) pairs.
__global__ __launch_bounds__(256) void argmax_finish_kernel(const Best* __restrict__ part, int chunks,
                                                            int32_t* __restrict__ argmax) {
    const int t = blockIdx.x;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    for (int c = threadIdx.x; c < chunks; c += 256) {
        const Best b = part[(int64_t)t * chunks + c];
        if (better(b.v, b.i, bv, bi)) {
            bv = b.v;
            bi = b.i;
        }
    }
    best16(bv, bi);
    __shared__ Best wb[16];
    if ((threadIdx.x & 15) == 0) wb[threadIdx.x >> 4] = Best{bv, bi};
    __syncthreads();
    if (threadIdx.x == 0) {
        Best b = wb[0];
        for (int w = 1; w < 16; w++)
            if (better(wb[w].v, wb[w].i, b.v, b.i)) b = wb[w];
        argmax[t] = b.i;
    }
}

bool linear_argmax_supported(int T, int N, int K) { return linear_mode(T, N, K) == kStream; }

int linear_argmax_chunks(int T, int N, int K) { return linear_argmax_supported(T, N, K) ? stream_grid(N) : 0; }

// Validated arguments. y may be null when amax is set; the argmax epilogue
// needs the streaming layout (linear_argmax_supported).
int linear_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, Best* amax,
                   int T, int N, int K, void* workspace, hipStream_t s) {
    int* cnt = static_cast<int*>(workspace);
    const size_t need = w4a8_linear_workspace(T, N, K);
    float* part = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
    switch (T) {
#define SPECV_CASE(n) \
    case n: return launch_T<n>(wq, ws, xq, xs, y, amax, part, cnt, N, K, s);
        SPECV_CASE(1) SPECV_CASE(2) SPECV_CASE(3) SPECV_CASE(4) SPECV_CASE(5) SPECV_CASE(6)
        SPECV_CASE(7) SPECV_CASE(8) SPECV_CASE(9) SPECV_CASE(10) SPECV_CASE(11) SPECV_CASE(12)
        SPECV_CASE(13) SPECV_CASE(14) SPECV_CASE(15) SPECV_CASE(16)
#undef SPECV_CASE
        default: return SPECV_E_SHAPE;
    }
}

}  // namespace specv

extern "C" int specv_time_next_linear(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return SPECV_E_INVAL;
    specv::g_time_start = static_cast<hipEvent_t>(start_event);
    specv::g_time_stop = static_cast<hipEvent_t>(stop_event);
    return SPECV_OK;
}

extern "C" size_t w4a8_linear_workspace(int32_t T, int32_t N, int32_t K) {
    using namespace specv;
    if (T < 1 || T > 16 || N < 1 || K < 32 || K % 32) return 0;
    const int mode = linear_mode(T, N, K);
    if (mode == kStream) return 0;
    return kCounterBytes + (size_t)mode * T * N * 4;
}

extern "C" int w4a8_linear_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                             float* y, int32_t T, int32_t N, int32_t K, void* workspace,
                             size_t workspace_bytes, void* stream) {
    using namespace specv;
    if (T < 1 || T > 16 || N < 0 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32)
        return SPECV_E_SHAPE;
    if ((int64_t)N * (K / 2) >= (int64_t)1 << 31) return SPECV_E_SHAPE;
    if (N == 0) return SPECV_OK;
    if (!wq || !ws || !xq || !xs || !y) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(ws, 2) || !aligned(xs, 4) || !aligned(y, 4))
        return SPECV_E_ALIGN;
    const size_t need = w4a8_linear_workspace(T, N, K);
    if (need && (!workspace || workspace_bytes < need)) return SPECV_E_WORKSPACE;
    if (need && !aligned(workspace, 256)) return SPECV_E_ALIGN;
    return linear_enqueue(wq, ws, xq, xs, y, nullptr, T, N, K, workspace, (hipStream_t)stream);
}

extern "C" size_t w4a8_linear_argmax_workspace(int32_t T, int32_t N, int32_t K) {
    using namespace specv;
    if (T < 1 || T > 16 || N < 1 || K < 32 || K % 32 || !linear_argmax_supported(T, N, K)) return 0;
    return (size_t)T * linear_argmax_chunks(T, N, K) * sizeof(Best);
}

extern "C" int w4a8_linear_argmax_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                                    float* y, int32_t* argmax, int32_t T, int32_t N, int32_t K, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    using namespace specv;
    if (T < 1 || T > 16 || N < 1 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32) return SPECV_E_SHAPE;
    if ((int64_t)N * (K / 2) >= (int64_t)1 << 31) return SPECV_E_SHAPE;
    if (!linear_argmax_supported(T, N, K)) return SPECV_E_SHAPE;
    if (!wq || !ws || !xq || !xs || !argmax) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(ws, 2) || !aligned(xs, 4) || !aligned(y, 4) ||
        !aligned(argmax, 4))
        return SPECV_E_ALIGN;
    const size_t need = w4a8_linear_argmax_workspace(T, N, K);
    if (!workspace || workspace_bytes < need) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 8)) return SPECV_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    Best* part = static_cast<Best*>(workspace);
    const int rc = linear_enqueue(wq, ws, xq, xs, y, part, T, N, K, nullptr, s);
    if (rc != SPECV_OK) return rc;
    hipLaunchKernelGGL(argmax_finish_kernel, dim3(T), dim3(256), 0, s, part, linear_argmax_chunks(T, N, K), argmax);
    return launch_status();
}
