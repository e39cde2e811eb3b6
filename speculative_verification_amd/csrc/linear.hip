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
//
// Work decomposition, three layouts chosen per shape:
//  narrow: a workgroup owns 16 rows and all K; its four waves take the four
//          slot quads (wave w: groups 16j + 4w + 0..3 in iteration j, 64
//          contiguous bytes per row), and the quad sums meet in LDS, where
//          the tree levels w = 4, 8 add them. Used when the matrix has few
//          rows: every CU gets work without splitting K. The four workgroups
//          of a 64-row block run on one XCD (they share scale lines).
//  wide:   a workgroup owns 64 rows (4 waves x 16) and all K; each wave takes
//          all four slot quads of its rows and finishes the tree in
//          registers. Used for tall matrices: 4x more rows share each staged
//          activation byte.
//  split:  64 rows and one of S K-slices (the Q = 4/S quads pQ..pQ+Q-1);
//          each slice reduces its own slots, and the last workgroup of a row
//          group to finish adds the S partials in tree order. The S
//          workgroups of a row group are numbered so that the hardware's
//          round-robin placement puts them on one XCD, whose L2 serves the
//          lines they share. Used when the staged activations of a whole row
//          would not fit in LDS.
// In all layouts a workgroup stages the activation codes it needs in LDS
// once, and every wave load covers 16 rows x 64 contiguous bytes.
//
// Integer dots. One v_mfma_i32_16x16x32_i8 computes, for 16 rows, the dots
// of one 8-input chunk of each group of a slot quad against up to four
// tokens: B (32x16) carries the weights, lane quarter q supplying the chunk of
// slot q of the quad for row l%16; A (16x32) carries the activations
// block-diagonally, row m = 4h+t holding token t's chunk of slot h in
// k-quarter h and zeros elsewhere. Output element (m, n) = (4h+t, row) is then
// exactly the chunk dot of row n, slot h, token t, and it lands in lane
// 16h + n, register t: the lane that loaded that row's group and scale. Four
// chunks accumulate in the int32 accumulator, giving the exact group dot.
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
// past G read zeros (an out-of-range offset in a ragged last iteration, no
// load in the padding iterations) against zero staged activations, so they
// add +0, which never changes a slot (a slot is never -0).
#include <hip/hip_ext.h>

#include "common.h"

namespace specv {

// Stages of weight loads kept in flight per wave. A narrow layout runs about
// one workgroup per CU, so it keeps many stages in flight to cover memory
// latency; the other layouts rely on several resident workgroups per CU.
#ifndef SPECV_NARROW_STAGES
#define SPECV_NARROW_STAGES 4
#endif
#ifndef SPECV_LINEAR_STAGES
#define SPECV_LINEAR_STAGES 2
#endif

template <int Q>
struct WStage {
    v4i w[Q];       // per slot quad: 16 bytes of nibbles (one group of one row)
    uint16_t s[Q];  // and its fp16 scale
};

__device__ __forceinline__ long mk64(int lo, int hi) {
    return (long)(((unsigned long)(unsigned)hi << 32) | (unsigned)lo);
}

// Staged activation layout in LDS: [t][j][QS*128 bytes] (the slice's groups
// of iteration j for token t) for j below J rounded up to whole blocks of P
// stages (zeros past the last group), followed by kZeroBytes of zeros that
// lanes whose A operand must be zero read instead.
enum { kNarrow = 0, kWide = 1 };  // modes; a split layout is MODE = S in {2, 4}
constexpr int kZeroBytes = 512;    // zero area after the staged activations

template <int T, int MODE>
__global__ __launch_bounds__(256) void w4a8_linear_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq,
    const float* __restrict__ xs, float* __restrict__ y, Best* __restrict__ amax, int write_y,
    float* __restrict__ part, int* __restrict__ cnt, int N, int K) {
    constexpr int S = MODE == kNarrow || MODE == kWide ? 1 : MODE;  // K-slices
    constexpr int QS = 4 / S;                        // slot quads staged per workgroup
    constexpr int Q = MODE == kNarrow ? 1 : QS;      // slot quads per wave
    constexpr int ROWS = MODE == kNarrow ? 16 : 64;  // rows per workgroup
    constexpr int TT = (T + 3) / 4;
    constexpr int P = MODE == kNarrow ? SPECV_NARROW_STAGES : SPECV_LINEAR_STAGES;
    extern __shared__ __attribute__((aligned(16))) int8_t act[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;         // row within the wave's 16; MFMA column n
    const int q = lane >> 4;         // slot within the quad; k-quarter of B
    const int h = (lane & 15) >> 2;  // slot of this lane's A row
    const int tp = lane & 3;         // token of this lane's A row within a tile
    const int G = K >> 5;
    const int J = (G + 15) >> 4;            // iterations of 16 groups
    const int JP = (J + P - 1) / P * P;     // staged iterations: whole blocks of P stages
    const int NG = (N + ROWS - 1) / ROWS;

    int rg, p;
    if (MODE == kNarrow) {
        // The four 16-row groups of a 64-row block share the 128-byte lines of
        // their group-major scales: number them so the hardware's round-robin
        // placement (workgroup b on XCD b mod 8) puts all four on one XCD,
        // whose L2 then fetches each line once.
        const int b = blockIdx.x, i = b >> 3;
        rg = 4 * ((i >> 2) * 8 + (b & 7)) + (i & 3);
        p = 0;
    } else if (S == 1) {
        rg = blockIdx.x;
        p = 0;
    } else {
        const int b = blockIdx.x, i = b >> 3;
        p = i % S;
        rg = (i / S) * 8 + (b & 7);
    }
    if (rg >= NG) return;
    const int row = rg * ROWS + (MODE == kNarrow ? 0 : wave * 16) + r;
    const bool row_ok = row < N;
    // first slot quad of this wave
    const int quad0 = MODE == kNarrow ? wave : p * QS;

    const auto rw = make_rsrc(wq, (uint32_t)((int64_t)N * (K / 2)));
    const auto rs = make_rsrc(wsg, (uint32_t)((int64_t)G * N * 2));
    const auto rx = make_rsrc(xq, (uint32_t)(T * K));

    // Stage loads carry almost no bounds logic. A row past N starts past the
    // end of the weights, so its loads return zeros. Iterations past the
    // last one (the pipeline's look-ahead and the padding of the last block)
    // load nothing: their stages are zeroed, and their staged activations are
    // zeros, so they add +0, which never changes a slot. Only in a ragged
    // last iteration (G not a multiple of 16) do lanes past G take an
    // out-of-range offset. The branches are uniform. Every offset is below
    // 2^32: the weights and scales are each under 2^31 bytes.
    const uint32_t wlane = (uint32_t)row * (uint32_t)(K / 2) + 16u * (uint32_t)(4 * quad0 + q);
    const uint32_t slane = ((uint32_t)(4 * quad0 + q) * (uint32_t)N + (uint32_t)row) * 2u;
    const bool ragged = (G & 15) != 0;
    auto load_fast = [&](WStage<Q>& st, int j) {  // j < J, and not a ragged last iteration
        const uint32_t wo = wlane + 256u * (uint32_t)j;
        const uint32_t so = slane + 32u * (uint32_t)N * (uint32_t)j;
#pragma unroll
        for (int qq = 0; qq < Q; qq++) {
            st.w[qq] = load16(rw, wo + 64u * (uint32_t)qq);
            st.s[qq] = load2(rs, so + 8u * (uint32_t)N * (uint32_t)qq);
        }
    };
    // Checked loads for the last block or two: past the last iteration the
    // whole wave takes the out-of-range bit (the loads return zeros without
    // touching memory); in a ragged last iteration, the lanes past G do.
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
    // the rounds' L2 round trips overlap. Inside every 8-input chunk the
    // codes are stored as inputs 0, 2, 4, 6, 1, 3, 5, 7: the order in which
    // the nibble decode below produces the weights, so the integer dot pairs
    // the same inputs (an exact integer sum in any order).
    const int nchunks = T * JP * QS * 8;  // 16-byte chunks
    // A narrow workgroup has its CU to itself and may hold 16 chunks per
    // round; chunks past the row are skipped by uniform branches, not loaded.
    constexpr int U = MODE == kNarrow && T >= 4 ? 16 : 8;
    auto stage_load = [&](v4i (&v)[U], int base) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (base + u * 256 >= nchunks) break;
            const int i = base + u * 256 + tid;
            const int c = i % (QS * 8);
            const int tj = i / (QS * 8);
            const int j = tj % JP;
            const int t = tj / JP;
            const int g = 16 * j + 4 * p * QS + (c >> 1);
            const bool ok = i < nchunks && g < G;
            v[u] = load16(rx, ((uint32_t)(t * K + 32 * g + 16 * (c & 1))) | ((uint32_t)!ok << 31));
        }
    };
    auto stage_store = [&](const v4i (&v)[U], int base) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (base + u * 256 >= nchunks) break;
            const int i = base + u * 256 + tid;
            if (i < nchunks) {
                const v4i a = v[u];
                const v4i e = {(int)__builtin_amdgcn_perm(a[1], a[0], 0x06040200u),
                               (int)__builtin_amdgcn_perm(a[1], a[0], 0x07050301u),
                               (int)__builtin_amdgcn_perm(a[3], a[2], 0x06040200u),
                               (int)__builtin_amdgcn_perm(a[3], a[2], 0x07050301u)};
                *reinterpret_cast<v4i*>(act + 16 * i) = e;
            }
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
    // zeros read by lanes whose A operand is zero (at most Q*128 bytes on)
    const int zero_off = nchunks * 16;
    if (tid < kZeroBytes / 16) *reinterpret_cast<v4i*>(act + zero_off + 16 * tid) = v4i{0, 0, 0, 0};
    __syncthreads();

    float acc[Q][T];
#pragma unroll
    for (int qq = 0; qq < Q; qq++)
#pragma unroll
        for (int t = 0; t < T; t++) acc[qq][t] = 0.0f;

    // A operand addresses: token t = 4tt + tp of slot h, advanced by one
    // staged iteration per j; lanes whose A row is zero stay on the zeros.
    int abase[TT], astep[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int t = 4 * tt + tp;
        const bool ok = q == h && t < T;
        abase[tt] = ok ? (t * JP * QS + (quad0 - p * QS)) * 128 + h * 32 : zero_off;
        astep[tt] = ok ? QS * 128 : 0;
    }
    auto compute = [&](const WStage<Q>& stg, int j) {
#pragma unroll
        for (int qq = 0; qq < Q; qq++) {
            // u = q + 8 in each nibble: flipping bit 3 gives q in 4-bit two's
            // complement; in the high half of a byte it is the int8 16q.
            // Even inputs come from the low nibbles, odd from the high ones.
            long b[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const unsigned W = (unsigned)stg.w[qq][c];
                const unsigned lo = ((W << 4) ^ 0x80808080u) & 0xF0F0F0F0u;  // inputs 0, 2, 4, 6
                const unsigned hi = (W ^ 0x80808080u) & 0xF0F0F0F0u;         // inputs 1, 3, 5, 7
                b[c] = mk64((int)lo, (int)hi);
            }
            v4i a0[TT], a1[TT];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                const int off = abase[tt] + j * astep[tt] + qq * 128;
                a0[tt] = *reinterpret_cast<const v4i*>(act + off);
                a1[tt] = *reinterpret_cast<const v4i*>(act + off + 16);
            }
            v4i d[TT];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) d[tt] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; c++)
#pragma unroll
                for (int tt = 0; tt < TT; tt++) {
                    const v4i& a = (c < 2) ? a0[tt] : a1[tt];
                    const long av = (c & 1) ? mk64(a[2], a[3]) : mk64(a[0], a[1]);
                    d[tt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, b[c], d[tt], 0, 0, 0);
                }
            const float s16 = (float)__builtin_bit_cast(_Float16, stg.s[qq]) * 0.0625f;
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    if (4 * tt + v < T) acc[qq][4 * tt + v] = acc[qq][4 * tt + v] + s16 * (float)d[tt][v];
        }
    };

    // P stages in flight. The steady loop's look-ahead loads are all plain
    // (in range, not a ragged last iteration); the last block or two take the
    // checked loads. Stages past the last iteration read zeros and their
    // staged activations are zeros, so the final block adds +0 for them. The
    // scheduling barriers keep each stage's use ahead of its refill.
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

    // Tree levels w = 1, 2 pair the four slots of a quad: lanes q^1, then q^2.
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

    // Optional argmax epilogue (amax != null): per token, the best
    // (value, lowest row) of the workgroup's rows goes to amax[t][rg]; the
    // outputs are written only when write_y is set.
    if (MODE == kNarrow) {  // levels w = 4, 8 across the four waves, in LDS
        __shared__ float red[4][T][16];
        if (q == 0)
#pragma unroll
            for (int t = 0; t < T; t++) red[wave][t][r] = val[0][t];
        __syncthreads();
        if (tid < 16 * T) {  // 16-lane groups: token t = tid / 16, row rr of the group
            const int t = tid >> 4, rr = tid & 15;
            const int orow = rg * ROWS + rr;
            const float v = xs[t] * ((red[0][t][rr] + red[1][t][rr]) + (red[2][t][rr] + red[3][t][rr]));
            if (orow < N && write_y) y[(int64_t)t * N + orow] = v;
            if (amax) {
                float bv = orow < N ? v : -__builtin_inff();
                int bi = orow < N ? orow : 0x7fffffff;
                best16(bv, bi);
                if (rr == 0) amax[(int64_t)t * NG + rg] = Best{bv, bi};
            }
        }
        return;
    }
    if (MODE == kWide) {  // levels w = 4, 8 inside the lane, then the token scale
        float vt[T];
#pragma unroll
        for (int t = 0; t < T; t++) vt[t] = xs[t] * ((val[0][t] + val[1 % Q][t]) + (val[2 % Q][t] + val[3 % Q][t]));
        if (q == 0 && row_ok && write_y)
#pragma unroll
            for (int t = 0; t < T; t++) y[(int64_t)t * N + row] = vt[t];
        if (amax) {  // lanes 0..15 of a wave hold its 16 rows (every quarter holds the same)
            __shared__ Best wb[4][T];
#pragma unroll
            for (int t = 0; t < T; t++) {
                float bv = row_ok ? vt[t] : -__builtin_inff();
                int bi = row_ok ? row : 0x7fffffff;
                best16(bv, bi);
                if (lane == 0) wb[wave][t] = Best{bv, bi};
            }
            __syncthreads();
            if (tid < T) {
                Best b = wb[0][tid];
#pragma unroll
                for (int w = 1; w < 4; w++)
                    if (better(wb[w][tid].v, wb[w][tid].i, b.v, b.i)) b = wb[w][tid];
                amax[(int64_t)tid * NG + rg] = b;
            }
        }
        return;
    }

    // S > 1: this slice's partial (level w = 4 inside the lane when Q = 2).
    // Partials and counters use device-scope relaxed atomic accesses: they
    // are coherent across the XCDs' separate L2 caches without a
    // device-scope fence (which would write back the whole L2). All partial
    // stores of the workgroup complete (s_waitcnt, then the barrier) before
    // its counter increment, so the workgroup that observes the final count
    // reads every partial.
    if (q == 0 && row_ok)
#pragma unroll
        for (int t = 0; t < T; t++)
            __hip_atomic_store(&part[((int64_t)p * T + t) * N + row],
                               (Q == 2) ? (val[0][t] + val[1 % Q][t]) : val[0][t], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
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

// Staged activation bytes of a workgroup in a given mode.
inline size_t linear_lds_bytes(int T, int K, int mode) {
    const int J = (K / 32 + 15) / 16;
    const int P = mode == kNarrow ? SPECV_NARROW_STAGES : SPECV_LINEAR_STAGES;
    const int JP = (J + P - 1) / P * P;
    const int qs = (mode == kNarrow || mode == kWide) ? 4 : 4 / mode;
    return (size_t)T * JP * qs * 128 + kZeroBytes;
}

constexpr size_t kLdsBudget = 150 * 1024;

// Layout for a shape: wide when there are enough 64-row groups to fill the
// chip, narrow otherwise, split when the staged activations of whole rows
// would not fit in LDS.
inline int linear_mode(int T, int N, int K) {
#ifdef SPECV_FORCE_LINEAR_MODE
    if (linear_lds_bytes(T, K, SPECV_FORCE_LINEAR_MODE) <= kLdsBudget) return SPECV_FORCE_LINEAR_MODE;
#endif
    const int NG64 = (N + 63) / 64;
    if (linear_lds_bytes(T, K, kWide) <= kLdsBudget) return NG64 >= 256 ? kWide : kNarrow;
    return linear_lds_bytes(T, K, 2) <= kLdsBudget && NG64 >= 256 ? 2 : 4;
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

template <int T, int MODE>
static int launch(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                  Best* amax, float* part, int* cnt, int N, int K, hipStream_t s) {
    const int write_y = y != nullptr;
    // Dynamic LDS above 64 KB must be enabled per kernel, up to what the
    // launch needs (the static LDS of the kernel counts towards the limit).
    static size_t lds_enabled = 64 * 1024;
    const size_t lds = linear_lds_bytes(T, K, MODE);
    if (lds > kLdsBudget) return SPECV_E_SHAPE;
    if (lds > lds_enabled) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&w4a8_linear_kernel<T, MODE>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        lds_enabled = lds;
    }
    const int grid = MODE == kNarrow ? ((N + 15) / 16 + 31) / 32 * 32
                     : MODE == kWide ? (N + 63) / 64
                                     : MODE * linear_row_groups_padded(N);
    if (g_time_start) {
        hipExtLaunchKernelGGL((w4a8_linear_kernel<T, MODE>), dim3(grid), dim3(256), lds, s, g_time_start,
                              g_time_stop, 0, wq, ws, xq, xs, y, amax, write_y, part, cnt, N, K);
        g_time_start = g_time_stop = nullptr;
    } else {
        hipLaunchKernelGGL((w4a8_linear_kernel<T, MODE>), dim3(grid), dim3(256), lds, s, wq, ws, xq, xs, y, amax,
                           write_y, part, cnt, N, K);
    }
    return launch_status();
}

template <int T>
static int launch_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                    Best* amax, float* part, int* cnt, int N, int K, hipStream_t s) {
    switch (linear_mode(T, N, K)) {
        case kNarrow: return launch<T, kNarrow>(wq, ws, xq, xs, y, amax, part, cnt, N, K, s);
        case kWide: return launch<T, kWide>(wq, ws, xq, xs, y, amax, part, cnt, N, K, s);
        case 2: return launch<T, 2>(wq, ws, xq, xs, y, nullptr, part, cnt, N, K, s);
        default: return launch<T, 4>(wq, ws, xq, xs, y, nullptr, part, cnt, N, K, s);
    }
}

// Finishes the argmax of each token from its row groups' partials.
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

bool linear_argmax_supported(int T, int N, int K) {
    const int mode = linear_mode(T, N, K);
    return mode == kNarrow || mode == kWide;
}

int linear_argmax_chunks(int T, int N, int K) {
    return linear_mode(T, N, K) == kNarrow ? (N + 15) / 16 : (N + 63) / 64;
}

// Validated arguments. y may be null when amax is set; the argmax epilogue
// needs the narrow or wide layout (linear_argmax_supported).
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
    if (mode == kNarrow || mode == kWide) return 0;
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
