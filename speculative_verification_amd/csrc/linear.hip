// W4A8 linear for T = 1..32 tokens on CDNA4 matrix cores.
//
// Operation (GPU-Resident Speculative Decoding for In-Browser LLM Inference
// with WebGPU, Small-Batch Verification Kernels and Implementation):
//   d[t][n][g] = sum_{k in group g} q(n,k) * xq[t][k]   exact int32
// per-token activation scales xs[t]:
//   p_g        = f32(scale[g][n]) * f32(d)               one rounding
//   y[t][n]    = xs[t] * R16(p_0 .. p_{G-1})             fixed order
// per-block activation scales xs[t][g] (one per 32 inputs):
//   p_g        = (f32(scale[g][n]) * xs[t][g]) * f32(d)  two roundings
//   y[t][n]    = R16(p_0 .. p_{G-1})
// R16: slot s in 0..15 accumulates the groups g = s, s+16, s+32, ... in
// increasing g from +0; the 16 slots are then added as a binary tree in
// index order (slot s += slot s+w for s divisible by 2w, w = 1, 2, 4, 8).
// An iteration j covers the 16 groups 16j .. 16j+15, one per slot; the 16
// slots form four quads of four.
//
// Work decomposition. About two workgroups per CU, each walking a list of
// 16-row tiles; its four waves take the four slot quads of every tile (wave
// w: groups 16j + 4w + 0..3, 64 contiguous bytes per row per iteration), and
// its weight loads run a fixed number of iterations ahead, across tile
// boundaries. A wave keeps its quarter of the activation codes in LDS after
// loading it with its first tile; when T x K is too large for LDS, the
// reload variant loads the quarter again with every tile instead.
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
// |16d| < 2^20). With per-token scales the weight scale is pre-divided by 16
// (exact: a power of two on a widened fp16 value), so f32(scale/16) *
// f32(16d) is the same real product as f32(scale) * f32(d) and rounds
// identically; with per-block scales d itself is recovered as 16d >> 4.
//
// Weights are read in the packed tile layout (pack.hip): the 16-byte group
// chunks of a 16-row tile follow each other group by group, so the load of
// one iteration by one wave (16 rows x 4 groups) is one contiguous kilobyte
// and a tile is one contiguous stream; the scales follow the same order.
//
// Ragged shapes. All global loads go through buffer resources, whose range
// check returns zeros. Rows past N are the zero rows that pad the last tile;
// groups past G read zeros (an out-of-range offset) against zero
// activations, so they add +0, which never changes a slot (a slot is never
// -0).
#include <hip/hip_ext.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace specv {

// Weight iterations in flight per wave, and workgroups per CU.
#ifndef SPECV_STREAM_STAGES
#define SPECV_STREAM_STAGES 4
#endif
#ifndef SPECV_STREAM_WGS_PER_CU
#define SPECV_STREAM_WGS_PER_CU 2
#endif

// Token buckets from this size scale each group dot with one fused
// multiply-add instead of a conversion and a multiply: the matrix
// instruction starts from a float bias, so the int32 result read as fp32 is
// exactly F = 12582912 + 16d (|16d| < 2^20), and fma(s, F, -s * 12582912)
// with s = scale / 16 is the exact product scale * d rounded once, as
// f32(scale) * f32(d) is (s * 12582912 has at most 13 significant bits, so
// it is exact). This needs finite scales: an infinite or NaN one gives NaN
// (smaller buckets keep the plain product, IEEE for every scale). Measured
// on MI355X, the 8B verify step at T = 8: 1049 -> 1033 us (median of five);
// a per-iteration test for non-finite scales in the wave, with the plain
// product as its branch, cost more than the fma saved.
constexpr int kFmaScaleMinT = 8;
constexpr int kScaleBiasBits = 0x4B400000;  // 12582912.0f
constexpr float kScaleBias = 12582912.0f;

// Token buckets up to this size take their integer dots from v_dot4_i32_i8
// instead of the matrix core (0: none). Measured on MI355X with rocprofv3
// on the 8B step's shapes: at T = 1 the two are within noise (965.5 against
// 981.1 us over a step's 129 launches), at T = 8 v_dot4 costs 1.26-1.80x
// per launch, so every bucket uses the matrix core.
#ifndef SPECV_DOT4_MAX_T
#define SPECV_DOT4_MAX_T 0
#endif

// The lane's 16 bytes of nibbles (32 inputs of one group) as int8 values
// 16q: b[0] holds inputs 0..15, b[1] inputs 16..31, each 8-input chunk in
// even-then-odd order (bytes 0, 2, 4, 6, then 1, 3, 5, 7).
__device__ __forceinline__ void decode_nibbles(const v4i w, v4i (&b)[2]) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const unsigned W = (unsigned)w[c];
        b[c >> 1][2 * (c & 1)] = (int)(((W << 4) ^ 0x80808080u) & 0xF0F0F0F0u);  // inputs 0, 2, 4, 6
        b[c >> 1][2 * (c & 1) + 1] = (int)((W ^ 0x80808080u) & 0xF0F0F0F0u);     // inputs 1, 3, 5, 7
    }
}

// Integer dots of one group per slot of a quad (see the header): w is the
// lane's 16 bytes of nibbles (32 inputs of its slot's group, row l%16); a0
// and a1 are the lane's A operands for inputs 0..15 and 16..31 of each token
// tile of 4. d[tt] receives c + 16 x the exact group dots.
template <int TT>
__device__ __forceinline__ void quad_dots(const v4i w, const v4i (&a0)[TT], const v4i (&a1)[TT], v4i (&d)[TT],
                                          const v4i c) {
    v4i b[2];
    decode_nibbles(w, b);
#pragma unroll
    for (int tt = 0; tt < TT; tt++) d[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[tt], b[0], c, 0, 0, 0);
#pragma unroll
    for (int tt = 0; tt < TT; tt++) d[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[tt], b[1], d[tt], 0, 0, 0);
}

// Tree levels w = 1, 2 of the four slots of a quad, which sit in the four
// 16-lane rows of a wave (slot q of the quad in row q): row q meets row
// q ^ 1, then row q ^ 2. A permlane swap of a value with itself returns, in
// a lane of the lower row (half) of a pair, its own value and the upper
// partner's, and in the upper row the lower partner's value and its own;
// each lane adds the partner's value to its own, so both lanes of a pair
// hold the same fp32 sum (a + b and b + a round alike). The exchanges of
// all tokens are issued together, in VALU registers, without LDS.
template <int T>
__device__ __forceinline__ void pair_rows(float (&s)[T]) {
    const int lane = threadIdx.x & 63;
    const bool odd_row = (lane >> 4) & 1, upper_half = lane >> 5;
#pragma unroll
    for (int t = 0; t < T; t++) {
        const unsigned u = __builtin_bit_cast(unsigned, s[t]);
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        s[t] = s[t] + __builtin_bit_cast(float, odd_row ? p[0] : p[1]);
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        const unsigned u = __builtin_bit_cast(unsigned, s[t]);
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        s[t] = s[t] + __builtin_bit_cast(float, upper_half ? p[0] : p[1]);
    }
}

// Activation codes of one 16-byte chunk (two 8-input chunks) in the
// even-then-odd order of the nibble decode: inputs 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ v4i even_odd(const v4i a) {
    return v4i{(int)__builtin_amdgcn_perm(a[1], a[0], 0x06040200u), (int)__builtin_amdgcn_perm(a[1], a[0], 0x07050301u),
               (int)__builtin_amdgcn_perm(a[3], a[2], 0x06040200u), (int)__builtin_amdgcn_perm(a[3], a[2], 0x07050301u)};
}

// Workgroup b of nwg walks the 16-row tiles b, b + nwg, b + 2 nwg, ... Its
// four waves take the four slot quads of
// every tile, so a wave only ever uses its own quarter of each token's
// activation codes: it loads that quarter together with a tile's weights,
// iteration by iteration, stores it in LDS in the MFMA operand order, and
// reads it back from there (for every later tile too, unless RELOAD). Slot pp
// of the load pipeline holds iterations pp, pp + P, ... of a tile, and in the
// tile's last block it is refilled with iteration pp of the next tile, so the
// stream does not drain between tiles. At the end of a tile the four quad
// sums of each row meet in LDS (tree levels w = 4, 8), and threads scale and
// store them, 16 rows per token. With an argmax (T <= 16), each finishing
// thread keeps the best of its rows over the tiles, and the workgroup writes
// one (value, lowest row) pair per token. T is the compiled token capacity;
// the call's token count Tr <= T (the 32-token bucket serves 17..32).
constexpr int kStreamZero = 64;  // zero bytes after the staged activations

template <int T, bool BS>
struct SStage {
    v4i w;                                 // 16 bytes of nibbles: one group of one row
    uint16_t s;                            // its fp16 scale
    v4i x[(T + 7) / 8];                    // activation quarter: 16 bytes per 8 tokens
    float xb[BS ? (4 * T + 63) / 64 : 1];  // block scales of the quarter's 4 groups, per token
};

// The activation rows of a fused linear (see ProdArgs), written as int8
// codes in the layout [t][j][quarter][128 bytes] (each 8-input chunk in
// even-then-odd order) with the token's scale in s_xs[t]. The arithmetic is
// the row kernels': RMSNorm takes ss = R16 over the squares x*x (16 lanes,
// each summing its slot in increasing k, then the lane tree), ms = ss / K,
// rs = 1 / sqrt(ms + eps), y = (x * rs) * w; SiLU rows are
// z = silu(gate) * up; both quantise with scale absmax / 127 and codes
// rint(v * 127 / absmax) clamped to +-127. Every row load of a token is
// issued before its first use, so a token costs about one memory round trip.
constexpr int kProdRegs = 4;       // float4 chunks per lane of a RMSNorm row kept in registers (K <= 1024)
constexpr int kRowsRegs = 6;       // float4 chunks per thread of a given row (K <= 6144)
// Given rows a fused linear quantises at most: every workgroup quantises all
// of them, and at four tokens that costs more than a row kernel's launch
// (measured on MI355X, 0.5B window: fused up to 2 tokens, width 2 went from
// 758 to 749 us per step; up to 4, width 4 lost 44 us per step).
constexpr int kRowsTokens = 2;

__device__ __forceinline__ float tree16_lanes(float v) {
#define SPECV_DPP_ADD(ctrl) \
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))
    SPECV_DPP_ADD(0xB1);
    SPECV_DPP_ADD(0x4E);
    SPECV_DPP_ADD(0x141);
    SPECV_DPP_ADD(0x140);
#undef SPECV_DPP_ADD
    return v;
}

// Lane l reads lane l ^ 1 (quad permutation 1, 0, 3, 2).
__device__ __forceinline__ int swap_pair(int v) { return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); }

// Maximum over the wave, uniform: each row of 16 lanes by DPP, then the four
// rows' values read as scalars. Every lane must be active.
__device__ __forceinline__ float wave_max(float v) {
#define SPECV_DPP_MAX(ctrl) \
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false)))
    SPECV_DPP_MAX(0xB1);
    SPECV_DPP_MAX(0x4E);
    SPECV_DPP_MAX(0x141);
    SPECV_DPP_MAX(0x140);
#undef SPECV_DPP_MAX
    const int b = __builtin_bit_cast(int, v);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}

__device__ __forceinline__ float max4(const float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Codes of inputs 4c .. 4c+3 (c = the calling lane's chunk). An 8-input
// chunk is stored evens first, so chunk 2m holds bytes 0, 4, 1, 5 of its
// 8-byte slot and chunk 2m + 1 bytes 2, 6, 3, 7: the even lane of a pair
// (c even, its neighbour lane holding c + 1) writes all 8 bytes. Both lanes
// of a pair must call this together, with chunks in range or not together.
__device__ __forceinline__ uint32_t code_of(float v, QuantScale qs) {
    return (uint32_t)(uint8_t)(int8_t)(int)quant_code(v, qs);
}

__device__ __forceinline__ void put_codes(int8_t* rowb, int c, const float4 y, QuantScale qs) {
    // this lane's evens (inputs 0, 2 of the chunk) and odds (1, 3), as byte pairs
    const uint32_t ev = code_of(y.x, qs) | code_of(y.z, qs) << 8;
    const uint32_t od = code_of(y.y, qs) | code_of(y.w, qs) << 8;
    const uint32_t ev2 = (uint32_t)swap_pair((int)ev);
    const uint32_t od2 = (uint32_t)swap_pair((int)od);
    if ((c & 1) == 0) {
        const int k0 = 4 * c;  // first input of the 8-input chunk
        const int gi = k0 >> 5;
        const int off = ((gi >> 4) * 4 + ((gi >> 2) & 3)) * 128 + (gi & 3) * 32 + (k0 & 31);
        *reinterpret_cast<uint2*>(rowb + off) = make_uint2(ev | ev2 << 16, od | od2 << 16);
    }
}

// Floats of a wave's RMSNorm buffer: the row itself (rows longer than
// 1024), or the squares of a row kept in registers as 16 slot rows of
// kSlotStride floats, positions past K / 16 zero (68, not 64: the 16
// summing lanes then read distinct banks).
constexpr int kSlotStride = 68;
__host__ __device__ inline int norm_row_floats(int K) {
    return K <= 1024 ? 16 * kSlotStride : 16 * (((K >> 4) + 3) & ~3);
}
// RMSNorm rows a fused linear produces at most, and at most spread over the
// whole workgroup (below that each wave takes its own tokens). Rows of K <=
// 1024 keep one slot area per token (4 per token of a wave), then 8 scales
// and 4 absmaxes per token.
constexpr int kNormMaxT = 8;
constexpr int kNormSpreadMaxT = 3;
__host__ __device__ inline int norm_scratch_floats(int T, int K) {
    return K <= 1024 ? (T + 3) / 4 * 4 * norm_row_floats(K) + 8 + 4 * kNormMaxT : 4 * norm_row_floats(K);
}

// Zero the staged row of token t (by one wave, or by the workgroup).
__device__ __forceinline__ void zero_row_lds(int8_t* act, int t, int JP, int first, int step) {
    v4i* row = reinterpret_cast<v4i*>(act + (size_t)t * JP * 512);
    for (int c = first; c < JP * 32; c += step) row[c] = v4i{0, 0, 0, 0};
}

// The 16 slot sums of a row's squares in the R16 order: slot s adds
// sq[s], sq[s + 16], ... in increasing k, then the lane tree. The squares
// sit transposed in the wave's LDS buffer (slot s at sq[s * stride ...]), so
// a slot lane reads its values as float4s, all issued before the adds.

// Sums of the squares of N rows in the fixed order, the slot areas of row n
// at sq + n * step: lane s < 16 adds the 64 positions of slot s in turn (the
// zeros past K / 16 leave a sum of squares unchanged, bit for bit), then the
// 16 slot sums meet in index order. The N chains interleave.
template <int N>
__device__ __forceinline__ void slot_sums(const float* sq, int step, int lane, float (&out)[N]) {
    float acc[N];
#pragma unroll
    for (int n = 0; n < N; n++) acc[n] = 0.0f;
    if (lane < 16) {
        constexpr int B = 16 / N;  // float4s of each row in flight per round
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += B) {
            float4 v[N][B];
#pragma unroll
            for (int n = 0; n < N; n++)
#pragma unroll
                for (int i = 0; i < B; i++)
                    v[n][i] = *reinterpret_cast<const float4*>(sq + n * step + lane * kSlotStride + 4 * (i0 + i));
#pragma unroll
            for (int i = 0; i < B; i++)
#pragma unroll
                for (int n = 0; n < N; n++) acc[n] = (((acc[n] + v[n][i].x) + v[n][i].y) + v[n][i].z) + v[n][i].w;
        }
    }
#pragma unroll
    for (int n = 0; n < N; n++) {
        const float a = tree16_lanes(acc[n]);
        out[n] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a)));
    }
}

// RMSNorm rows of up to kNormSpreadMaxT tokens, K <= 1024: thread i takes
// chunk i (inputs 4i .. 4i+3) of every token, so the per-value work is
// spread over the workgroup. The squares meet in LDS, where wave t sums token
// t's slots; its scale and the four waves' absmaxes are exchanged there too.
// (From 4 tokens on, each wave's own serial chains per token, its absmax and
// the scale's division, cost more than the spread saves.)
template <int T, typename Issue>
__device__ void produce_norm_spread(const ProdArgs& pa, int Tr, int live, int K, int JP, int8_t* act, float* s_xs,
                                    float* scratch, Issue&& issue) {
    static_assert(T <= kNormSpreadMaxT, "one token per summing wave");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid;
    const bool in = c < (K >> 2);
    const bool wb = pa.h_out && pa.b && blockIdx.x == 0;
    const uint32_t rowb = (uint32_t)(Tr * K * 4);
    const auto ra = make_rsrc(pa.a, rowb);
    const auto rd = make_rsrc(pa.b ? pa.b : pa.a, pa.b ? rowb : 0u);
    const auto rwn = make_rsrc(pa.w, (uint32_t)(K * 4));
    float4 x[T], d[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
        const uint32_t off = ((uint32_t)(t * K + 4 * c) * 4u) | (t < Tr && in ? 0u : kOOB);
        x[t] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
        d[t] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
    }
    const float4 wv = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(rwn, ((uint32_t)c * 16u) | (in ? 0u : kOOB), 0, 0));
    issue();
    const auto rh = make_rsrc(pa.h_out, wb ? rowb : 0u);  // the summed residual, by workgroup 0
    float* ex = scratch + T * 16 * kSlotStride;            // scales [8], absmaxes [T][4]
    for (int t = wave; t < T; t += 4) {
        zero_row_lds(act, t, JP, lane, 64);
        if (lane == 0) s_xs[t] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        if (t >= Tr || t >= live) continue;
        float4& v = x[t];
        if (pa.b) v = make_float4(v.x + d[t].x, v.y + d[t].y, v.z + d[t].z, v.w + d[t].w);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rh,
                                               ((uint32_t)(t * K + 4 * c) * 4u) | (in ? 0u : kOOB), 0, 0);
        // slots (4c & 15) + e, position c >> 2; zero past K
        float* q = scratch + t * 16 * kSlotStride + (4 * c & 15) * kSlotStride + (c >> 2);
        q[0] = v.x * v.x;
        q[kSlotStride] = v.y * v.y;
        q[2 * kSlotStride] = v.z * v.z;
        q[3 * kSlotStride] = v.w * v.w;
    }
    __syncthreads();
    if (wave < T && wave < Tr && wave < live) {
        float ss[1];
        slot_sums<1>(scratch + wave * 16 * kSlotStride, 0, lane, ss);
        if (lane == 0) ex[wave] = 1.0f / sqrtf(ss[0] / (float)K + pa.eps);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; t++) {
        if (t >= Tr || t >= live) continue;
        const float rs = ex[t];
        float4& v = x[t];
        v = make_float4((v.x * rs) * wv.x, (v.y * rs) * wv.y, (v.z * rs) * wv.z, (v.w * rs) * wv.w);
        const float amax = wave_max(in ? max4(v) : 0.0f);
        if (lane == 0) ex[8 + 4 * t + wave] = amax;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; t++) {
        if (t >= Tr || t >= live) continue;
        const float* m4 = ex + 8 + 4 * t;
        const float m = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        const QuantScale qs = quant_scale(m);
        if (tid == 0) s_xs[t] = m == 0.0f ? 0.0f : m / 127.0f;
        if (in) put_codes(act + (size_t)t * JP * 512, c, x[t], qs);
    }
}

// RMSNorm rows: wave w takes tokens w, w + 4, ... Rows of up to 1024 values
// live in registers, every load of the wave's tokens issued up front; longer
// rows go through the wave's LDS row and read the weight twice.
template <int T, typename Issue>
__device__ void produce_norm(const ProdArgs& pa, int Tr, int live, int K, int JP, int8_t* act, float* s_xs,
                             float* scratch, Issue&& issue) {
    constexpr int TPW = (T + 3) / 4;  // tokens per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K4 = K >> 2;
    const bool wb = pa.h_out && pa.b && blockIdx.x == 0;
    static_assert(T <= kNormMaxT, "RMSNorm rows of at most kNormMaxT tokens");
    float* xr = scratch + (size_t)wave * norm_row_floats(K);
    if constexpr (T <= kNormSpreadMaxT) {
        if (K4 <= 64 * kProdRegs) return produce_norm_spread<T>(pa, Tr, live, K, JP, act, s_xs, scratch, issue);
    }
    if (K4 <= 64 * kProdRegs) {
        // Every row load is issued, out of range where there is no value (a
        // token past Tr, a chunk past K, no residual), so the compiler counts
        // them, and before the first weights: the rows are then waited for
        // alone, while the weights stream (loads complete in order).
        const uint32_t rowb = (uint32_t)(Tr * K * 4);
        const auto ra = make_rsrc(pa.a, rowb);
        const auto rd = make_rsrc(pa.b ? pa.b : pa.a, pa.b ? rowb : 0u);
        const auto rwn = make_rsrc(pa.w, (uint32_t)(K * 4));
        float4 x[TPW][kProdRegs], d[TPW][kProdRegs], wv[kProdRegs];
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int t = wave + 4 * u;
#pragma unroll
            for (int i = 0; i < kProdRegs; i++) {
                const int c = lane + 64 * i;
                const uint32_t off = ((uint32_t)(t * K + 4 * c) * 4u) | (t < T && t < Tr && c < K4 ? 0u : kOOB);
                x[u][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
                d[u][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < kProdRegs; i++) {
            const int c = lane + 64 * i;
            wv[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rwn, ((uint32_t)c * 16u) | (c < K4 ? 0u : kOOB), 0, 0));
        }
        issue();
        const auto rh = make_rsrc(pa.h_out, wb ? rowb : 0u);  // the summed residual, by workgroup 0
        for (int t = wave; t < T; t += 4) {
            zero_row_lds(act, t, JP, lane, 64);
            if (lane == 0) s_xs[t] = 0.0f;
        }
        // In phases over the wave's tokens, each in its own slot area, so
        // that their serial chains (slot sums, absmaxes) interleave. A token
        // past T, Tr or the live count goes through them on zeros, or on its
        // row, and leaves nothing behind.
        constexpr int kArea = 4 * 16 * kSlotStride;  // token wave + 4u: area u of the wave's
        float* xa = scratch + (size_t)wave * 16 * kSlotStride;
        bool ok[TPW];
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int t = wave + 4 * u;
            ok[u] = t < T && t < Tr && t < live;
            // every chunk of the 1024 positions, zero past K (its loads were out of range)
#pragma unroll
            for (int i = 0; i < kProdRegs; i++) {
                const int c = lane + 64 * i;
                float4& v = x[u][i];
                if (pa.b) v = make_float4(v.x + d[u][i].x, v.y + d[u][i].y, v.z + d[u][i].z, v.w + d[u][i].w);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(v4i, v), rh, ((uint32_t)(t * K + 4 * c) * 4u) | (ok[u] && c < K4 ? 0u : kOOB),
                    0, 0);
                // inputs 4c .. 4c+3: slots (4c & 15) + e, position 4c >> 4 within the slot
                float* q = xa + u * kArea + (4 * c & 15) * kSlotStride + (c >> 2);
                q[0] = v.x * v.x;
                q[kSlotStride] = v.y * v.y;
                q[2 * kSlotStride] = v.z * v.z;
                q[3 * kSlotStride] = v.w * v.w;
            }
        }
        float ss[TPW], am[TPW];
        slot_sums<TPW>(xa, kArea, lane, ss);
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const float rs = 1.0f / sqrtf(ss[u] / (float)K + pa.eps);
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < kProdRegs; i++) {
                float4& v = x[u][i];
                v = make_float4((v.x * rs) * wv[i].x, (v.y * rs) * wv[i].y, (v.z * rs) * wv[i].z,
                                (v.w * rs) * wv[i].w);
                amax = fmaxf(amax, lane + 64 * i < K4 ? max4(v) : 0.0f);
            }
            am[u] = wave_max(amax);
        }
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            if (!ok[u]) continue;
            const int t = wave + 4 * u;
            const QuantScale qs = quant_scale(am[u]);
            if (lane == 0) s_xs[t] = am[u] == 0.0f ? 0.0f : am[u] / 127.0f;
#pragma unroll
            for (int i = 0; i < kProdRegs; i++)
                if (lane + 64 * i < K4) put_codes(act + (size_t)t * JP * 512, lane + 64 * i, x[u][i], qs);
        }
        return;
    }
    issue();
    for (int t = wave; t < T; t += 4) {
        zero_row_lds(act, t, JP, lane, 64);
        if (lane == 0) s_xs[t] = 0.0f;
    }
    for (int t = wave; t < T && t < Tr && t < live; t += 4) {
        const float* ar = pa.a + (size_t)t * K;
        const float* br = pa.b ? pa.b + (size_t)t * K : nullptr;
        int8_t* rowb = act + (size_t)t * JP * 512;
        for (int c = lane; c < K4; c += 64) {
            float4 v = *reinterpret_cast<const float4*>(ar + 4 * c);
            if (br) {
                const float4 d = *reinterpret_cast<const float4*>(br + 4 * c);
                v = make_float4(v.x + d.x, v.y + d.y, v.z + d.z, v.w + d.w);
                if (wb) *reinterpret_cast<float4*>(pa.h_out + (size_t)t * K + 4 * c) = v;
            }
            *reinterpret_cast<float4*>(xr + 4 * c) = v;
        }
        float acc = 0.0f;
        if (lane < 16)
            for (int k = lane; k < K; k += 16) acc = acc + xr[k] * xr[k];
        acc = tree16_lanes(acc);
        const float ss = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, acc)));
        const float rs = 1.0f / sqrtf(ss / (float)K + pa.eps);
        auto value4 = [&](int c) {
            const float4 x = *reinterpret_cast<const float4*>(xr + 4 * c);
            const float4 wv = *reinterpret_cast<const float4*>(pa.w + 4 * c);
            return make_float4((x.x * rs) * wv.x, (x.y * rs) * wv.y, (x.z * rs) * wv.z, (x.w * rs) * wv.w);
        };
        float amax = 0.0f;
        for (int c = lane; c < K4; c += 64) amax = fmaxf(amax, max4(value4(c)));
        amax = wave_max(amax);
        const QuantScale qs = quant_scale(amax);
        if (lane == 0) s_xs[t] = amax == 0.0f ? 0.0f : amax / 127.0f;
        for (int c = lane; c < K4; c += 64) put_codes(rowb, c, value4(c), qs);
    }
}

// Given rows (at most kRowsTokens): the whole workgroup, every load issued
// up front, values in registers, each token's absmax met in LDS.
template <int T, typename Issue>
__device__ void produce_given(const ProdArgs& pa, int Tr, int live, int K, int JP, int8_t* act, float* s_xs,
                              float* part, Issue&& issue) {
    constexpr int TS = T < kRowsTokens ? T : kRowsTokens;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K4 = K >> 2;
    // every row load issued (out of range where there is no value), then the
    // first weights, as for the RMSNorm rows
    const auto ra = make_rsrc(pa.a, (uint32_t)(Tr * K * 4));
    float4 zv[TS][kRowsRegs];
#pragma unroll
    for (int t = 0; t < TS; t++) {
#pragma unroll
        for (int i = 0; i < kRowsRegs; i++) {
            const int c = tid + 256 * i;
            const uint32_t off = ((uint32_t)(t * K + 4 * c) * 4u) | (t < Tr && c < K4 ? 0u : kOOB);
            zv[t][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
        }
    }
    issue();
    for (int t = 0; t < T; t++) zero_row_lds(act, t, JP, tid, 256);
    if (tid < T) s_xs[tid] = 0.0f;
    float amax[TS];
#pragma unroll
    for (int t = 0; t < TS; t++) {
        amax[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < kRowsRegs; i++)
            if (t < Tr && t < live && tid + 256 * i < K4) amax[t] = fmaxf(amax[t], max4(zv[t][i]));
        amax[t] = wave_max(amax[t]);
        if (lane == 0) part[4 * t + wave] = amax[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TS; t++) {
        if (t >= Tr || t >= live) continue;
        const float m = fmaxf(fmaxf(part[4 * t], part[4 * t + 1]), fmaxf(part[4 * t + 2], part[4 * t + 3]));
        const QuantScale qs = quant_scale(m);
        if (tid == 0) s_xs[t] = m == 0.0f ? 0.0f : m / 127.0f;
        int8_t* rowb = act + (size_t)t * JP * 512;
#pragma unroll
        for (int i = 0; i < kRowsRegs; i++)
            if (tid + 256 * i < K4) put_codes(rowb, tid + 256 * i, zv[t][i], qs);
    }
}

// All rows of the step; tokens past Tr or the live count, and padding
// groups, stay zero. Each producer issues its row loads before it zeroes the
// staged rows, so the two overlap.
template <int T, int PROD, typename Issue>
__device__ void produce_rows(const ProdArgs& pa, int Tr, int K, int JP, int8_t* act, float* s_xs, float* scratch,
                             Issue&& issue) {
    const bool done = pa.ctrl->done != 0;
    const int live = done ? 0 : pa.ctrl->n_nodes;
    if constexpr (PROD == kProdNorm)
        produce_norm<T>(pa, Tr, live, K, JP, act, s_xs, scratch, issue);
    else
        produce_given<T>(pa, Tr, live, K, JP, act, s_xs, scratch, issue);
}

template <int T, int P, bool AMAX, bool BS, bool RELOAD, int PROD>
__global__ __launch_bounds__(256) void w4a8_linear_stream_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsg, const int8_t* __restrict__ xq, int N, int K,
    int nwg, int Tr, const float* __restrict__ xs, float* __restrict__ y, int write_y, Best* __restrict__ amax,
    const ProdArgs pa) {
    constexpr int TT = (T + 3) / 4;
    constexpr int TX = (T + 7) / 8;
    constexpr int XB = (4 * T + 63) / 64;  // block-scale loads per lane and iteration
    constexpr int FP = (16 * T + 255) / 256;  // finishing passes: 16 rows per token, 256 threads
    extern __shared__ __attribute__((aligned(16))) int8_t act[];
    __shared__ float red[2][4][T][16];
    __shared__ float s_xs[PROD != kProdNone ? T : 1];  // token scales of produced rows
    static_assert(!AMAX || T <= 16, "the argmax keeps one token per finishing thread");
    static_assert(PROD == kProdNone || (!BS && !RELOAD), "produced rows are kept in LDS, per-token scales");

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
    const int JA = RELOAD ? 1 : JP;      // iterations kept in LDS
    const int NT = (N + 15) >> 4;
    // Workgroup b takes tiles b, b + nwg, ...: the workgroups in flight
    // read neighbouring stretches of the packed matrix, front to back.
    const int b = blockIdx.x;
    const int v = b;
    const int ntiles = v < NT ? (NT - v + nwg - 1) / nwg : 0;

    // With the argmax, thread (ft, fr) finishes row fr of token ft.
    const int ft = tid >> 4, fr = tid & 15;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    if (ntiles == 0) {
        if (AMAX && ft < Tr && fr == 0) amax[(int64_t)ft * nwg + b] = Best{bv, bi};
        return;
    }
    float fxs[FP];
#pragma unroll
    for (int k = 0; k < FP; k++) {
        const int t = (tid + 256 * k) >> 4;
        fxs[k] = !BS && PROD == kProdNone && t < Tr ? xs[t] : 0.0f;
    }

    const auto rw = make_rsrc(wq, (uint32_t)packed_weight_bytes(N, K));
    // From kFmaScaleMinT tokens (finite scales) the weight loads go through
    // a resource per tile and need no per-lane masks: measured on MI355X, the
    // 8B verify step at T = 8 took 1025 against 1029.6 us (median of five,
    // two runs each), 7.51-7.52 against 7.60-7.69 us per linear launch.
    constexpr bool LEAN = !BS && T >= kFmaScaleMinT && T > SPECV_DOT4_MAX_T;
    const uint32_t wbytes = (uint32_t)packed_weight_bytes(N, K), sbytes = (uint32_t)packed_scale_bytes(N, K);
    const auto rs = make_rsrc(wsg, (uint32_t)packed_scale_bytes(N, K));
    const auto rx = make_rsrc(xq, (uint32_t)(Tr * K));
    const auto rb = make_rsrc(xs, BS ? (uint32_t)(Tr * G * 4) : 0u);
    const uint32_t lq = 4u * wave + q;  // group of this lane within an iteration
    const uint32_t wlane = (lq * 16u + (uint32_t)r) * 16u, slane = (lq * 16u + (uint32_t)r) * 2u;
    const int xc = lane & 7;            // 16-byte chunk of the quarter this lane loads
    const uint32_t xlane = 32u * (4u * wave + (xc >> 1)) + 16u * (xc & 1);

    // One iteration j of a tile: the lane's 16 bytes of nibbles and scale,
    // and with the activations, 16 bytes of codes per 8 tokens (and with block
    // scales, one scale per lane for up to 64 (token, group) pairs). Every
    // load is issued unconditionally, so the compiler counts them statically:
    // a group past G (a ragged or padding iteration), a token past Tr and a
    // tile past the list take the out-of-range bit, and all of these read
    // zeros (rows past N are zero rows of the packed layout). Offsets stay
    // below 2^32 (the packed weights and scales are each under 2^31 bytes),
    // or have the out-of-range bit set.
    auto load = [&](SStage<T, BS>& st, int tile, int j, bool with_act, uint32_t past) {
        if constexpr (LEAN) {
            // the tile's own resource (its groups from the first on): the
            // lane part of the offset is fixed and j adds a constant; groups
            // past G meet zero activations, so they need no mask (they read
            // the next tile's finite weights, or zeros past the end)
            const uint32_t t0 = (uint32_t)tile * (uint32_t)G;
            const bool live_tile = (uint32_t)tile < (uint32_t)NT && past == 0u;
            const auto rwt = make_rsrc(wq + (size_t)t0 * 256u, live_tile ? wbytes - t0 * 256u : 0u);
            const auto rst = make_rsrc(wsg + (size_t)t0 * 16u, live_tile ? sbytes - t0 * 32u : 0u);
            st.w = load16_stream(rwt, wlane + 4096u * (uint32_t)j);
            st.s = load2_stream(rst, slane + 512u * (uint32_t)j);
        } else {
            const uint32_t bad = ((16 * j + (int)lq >= G) ? kOOB : 0u) | past;
            const uint32_t chunk = ((uint32_t)tile * (uint32_t)G + 16u * (uint32_t)j + lq) * 16u + (uint32_t)r;
            st.w = load16_stream(rw, (chunk * 16u) | bad);
            st.s = load2_stream(rs, (chunk * 2u) | bad);
        }
        if (with_act) {
#pragma unroll
            for (int x = 0; x < TX; x++) {
                const int xt = (lane >> 3) + 8 * x;
                const bool ok = xt < Tr && 16 * j + 4 * wave + (xc >> 1) < G;
                st.x[x] = load16(rx, ((uint32_t)(xt * K + 512 * j) + xlane) | (ok ? 0u : kOOB));
            }
            if constexpr (BS) {
#pragma unroll
                for (int x = 0; x < XB; x++) {
                    const int e = lane + 64 * x;  // (token e >> 2, group 16j + 4 wave + (e & 3))
                    const int g = 16 * j + 4 * wave + (e & 3);
                    const bool ok = (e >> 2) < Tr && g < G;
                    st.xb[x] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(
                                   rb, ((uint32_t)((e >> 2) * G + g) * 4u) | (ok ? 0u : kOOB), 0, 0));
                }
            }
        }
    };
    // LDS: activation chunks as [t][ja][wave][128 bytes] (ja = j, or 0 when
    // reloading), the zero bytes, then with block scales [ja][wave][slot][T]
    // floats. Only this wave reads what it stores, and a wave's LDS accesses
    // complete in order, so no barrier is needed.
    const int zero_off = T * JA * 512;
    float* xbl = reinterpret_cast<float*>(act + zero_off + kStreamZero);
    auto put_act = [&](const SStage<T, BS>& st, int j) {
        const int ja = RELOAD ? 0 : j;
#pragma unroll
        for (int x = 0; x < TX; x++) {
            const int xt = (lane >> 3) + 8 * x;
            if (xt < T) *reinterpret_cast<v4i*>(act + ((xt * JA + ja) * 4 + wave) * 128 + 16 * xc) = even_odd(st.x[x]);
        }
        if constexpr (BS) {
#pragma unroll
            for (int x = 0; x < XB; x++) {
                const int e = lane + 64 * x;
                if ((e >> 2) < T) xbl[((ja * 4 + wave) * 4 + (e & 3)) * T + (e >> 2)] = st.xb[x];
            }
        }
    };

    // A operand addresses: token t = 4tt + tp of slot h, advanced by one
    // iteration per j; lanes whose A row is zero stay on the zero bytes.
    int abase[TT], astep[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int t = 4 * tt + tp;
        const bool ok = q == h && t < T;
        abase[tt] = ok ? (t * JA * 4 + wave) * 128 + h * 32 : zero_off;
        astep[tt] = ok && !RELOAD ? 512 : 0;
    }
    // dv[t]: 16 x the exact dot of row r, group 16j + 4 wave + q, token t
    auto compute = [&](const SStage<T, BS>& st, int j, float (&acc)[T]) {
        int dv[T];
        if constexpr (T <= SPECV_DOT4_MAX_T) {
            // each lane dots its own row's group with every token's 32 codes
            // (the lanes of a slot read the same LDS words)
            v4i b[2];
            decode_nibbles(st.w, b);
#pragma unroll
            for (int t = 0; t < T; t++) {
                const int off = ((t * JA + (RELOAD ? 0 : j)) * 4 + wave) * 128 + 32 * q;
                const v4i x0 = *reinterpret_cast<const v4i*>(act + off);
                const v4i x1 = *reinterpret_cast<const v4i*>(act + off + 16);
                int a = 0;
#pragma unroll
                for (int e = 0; e < 4; e++) a = __builtin_amdgcn_sdot4(b[0][e], x0[e], a, false);
#pragma unroll
                for (int e = 0; e < 4; e++) a = __builtin_amdgcn_sdot4(b[1][e], x1[e], a, false);
                dv[t] = a;
            }
        } else {
            v4i a0[TT], a1[TT], d[TT];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                const int off = abase[tt] + j * astep[tt];
                a0[tt] = *reinterpret_cast<const v4i*>(act + off);
                a1[tt] = *reinterpret_cast<const v4i*>(act + off + 16);
            }
            constexpr int cb = !BS && T >= kFmaScaleMinT ? kScaleBiasBits : 0;
            quad_dots<TT>(st.w, a0, a1, d, v4i{cb, cb, cb, cb});
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (4 * tt + u < T) dv[4 * tt + u] = d[tt][u];
        }
        if constexpr (BS) {
            // s = f32(scale) * xs[t][g], then s * f32(d), with d = 16d >> 4 exactly
            const float ws32 = (float)__builtin_bit_cast(_Float16, st.s);
            const float* xb = xbl + (((RELOAD ? 0 : j) * 4 + wave) * 4 + q) * T;
#pragma unroll
            for (int t = 0; t < T; t++) acc[t] = acc[t] + (ws32 * xb[t]) * (float)(dv[t] >> 4);
        } else if constexpr (T >= kFmaScaleMinT && T > SPECV_DOT4_MAX_T) {
            // dv[t]: the bits of F = 12582912 + 16d
            const float s16 = (float)__builtin_bit_cast(_Float16, st.s) * 0.0625f;
            const float c = -(s16 * kScaleBias);
#pragma unroll
            for (int t = 0; t < T; t++) acc[t] = acc[t] + __builtin_fmaf(s16, __builtin_bit_cast(float, dv[t]), c);
        } else {
            const float s16 = (float)__builtin_bit_cast(_Float16, st.s) * 0.0625f;
#pragma unroll
            for (int t = 0; t < T; t++) acc[t] = acc[t] + s16 * (float)dv[t];
        }
    };

    SStage<T, BS> st[P];
    auto issue_first = [&]() {  // the first P iterations of the first tile
#pragma unroll
        for (int pp = 0; pp < P; pp++) {
            load(st[pp], v, pp, PROD == kProdNone, 0u);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (PROD == kProdNone) issue_first();
    if (tid < kStreamZero / 16) *reinterpret_cast<v4i*>(act + zero_off + 16 * tid) = v4i{0, 0, 0, 0};
    if constexpr (PROD != kProdNone)  // the rows; the first weights go out right after their loads
        produce_rows<T, PROD>(pa, Tr, K, JP, act, s_xs,
                              reinterpret_cast<float*>(act + zero_off + kStreamZero + (BS ? JA * 64 * T : 0)),
                              issue_first);
    __syncthreads();

    auto run_tile = [&](auto first_tag, int k, float (&acc)[T]) {
        constexpr bool WITH_ACT = decltype(first_tag)::value || RELOAD;  // this tile brings its activations
        const int tile = v + k * nwg;
        int j0 = 0;
        for (; j0 + P < JP; j0 += P) {
#pragma unroll
            for (int pp = 0; pp < P; pp++) {
                if (WITH_ACT) put_act(st[pp], j0 + pp);
                compute(st[pp], j0 + pp, acc);
                __builtin_amdgcn_sched_barrier(0);
                load(st[pp], tile, j0 + pp + P, WITH_ACT, 0u);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const uint32_t past = k + 1 < ntiles ? 0u : kOOB;
#pragma unroll
        for (int pp = 0; pp < P; pp++) {
            if (WITH_ACT) put_act(st[pp], j0 + pp);
            compute(st[pp], j0 + pp, acc);
            __builtin_amdgcn_sched_barrier(0);
            load(st[pp], tile + nwg, pp, RELOAD, past);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // End of a tile: levels w = 1, 2 pair the four slots of a quad (lanes
    // q ^ 1, q ^ 2), levels w = 4, 8 the four waves' quads, in LDS. The
    // reduction buffer alternates between tiles: a tile's reads of it end
    // before any thread passes the next tile's barrier.
    auto finish_tile = [&](int k, const float (&acc)[T], int buf) {
        const int tile = v + k * nwg;
        float s[T];
#pragma unroll
        for (int t = 0; t < T; t++) s[t] = acc[t];
        pair_rows<T>(s);
        if (q == 0) {
#pragma unroll
            for (int t = 0; t < T; t++) red[buf][wave][t][r] = s[t];
        }
        __syncthreads();
        auto out = [&](int t, int rr, int kk) {  // output of row 16 tile + rr for token t
            const float sum = (red[buf][0][t][rr] + red[buf][1][t][rr]) + (red[buf][2][t][rr] + red[buf][3][t][rr]);
            return BS ? sum : (PROD != kProdNone ? s_xs[t] : fxs[kk]) * sum;
        };
        if (!AMAX && pa.epi == kEpiSiluPairs) {
            // rows rr < 8 of the tile are gate rows 8 tile + rr, rows rr + 8
            // the up rows of the same index: z = silu(g) * u
#pragma unroll
            for (int kk = 0; kk < FP; kk++) {
                const int idx = tid + 256 * kk;
                const int t = idx >> 4, rr = idx & 15;
                if (t < Tr && rr < 8 && 16 * tile < N) {
                    const float g = out(t, rr, kk), u = out(t, rr + 8, kk);
                    y[(int64_t)t * (N >> 1) + 8 * tile + rr] = silu(g) * u;
                }
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < FP; kk++) {
                const int idx = tid + 256 * kk;
                const int t = idx >> 4, rr = idx & 15;
                const int row = 16 * tile + rr;
                if (t < Tr && row < N) {
                    const float val = out(t, rr, kk);
                    if (!AMAX || write_y) y[(int64_t)t * N + row] = val;
                    if (AMAX && better(val, row, bv, bi)) {
                        bv = val;
                        bi = row;
                    }
                }
            }
        }
    };
    if constexpr (PROD == kProdNone) {  // the first tile brings the activations
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; t++) acc[t] = 0.0f;
        run_tile(std::true_type{}, 0, acc);
        finish_tile(0, acc, 0);
    }
    for (int k = PROD == kProdNone ? 1 : 0; k < ntiles; k++) {
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; t++) acc[t] = 0.0f;
        run_tile(std::false_type{}, k, acc);
        finish_tile(k, acc, k & 1);
    }
    if (AMAX && ft < Tr) {
        best16(bv, bi);
        if (fr == 0) amax[(int64_t)ft * nwg + b] = Best{bv, bi};
    }
}

// ---------------------------------------------------------------- host

constexpr size_t kLdsBudget = 150 * 1024;

// Dynamic LDS of a workgroup (its tile reduction buffer, 512T bytes, is
// static): the activation quarters of JA iterations, the zero bytes, and the
// block scales.
inline size_t stream_lds_bytes(int T, int K, bool bs, bool reload, int P = SPECV_STREAM_STAGES) {
    const int J = (K / 32 + 15) / 16;
    const int JA = reload ? 1 : (J + P - 1) / P * P;
    return (size_t)T * JA * 512 + kStreamZero + (bs ? (size_t)JA * 64 * T : 0);
}
// LDS of a producer: one row per wave (RMSNorm), the absmax exchange (SiLU).
inline size_t prod_scratch_bytes(int prod, int T, int K) {
    return prod == kProdNorm ? (size_t)4 * norm_scratch_floats(T, K) : prod == kProdRows ? 16 * kRowsTokens : 0;
}
// Whether the activations of every iteration fit beside the reduction buffer.
inline bool stream_keeps(int T, int K, bool bs) {
    return stream_lds_bytes(T, K, bs, false) + (size_t)T * 512 <= kLdsBudget;
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

// Workgroups of a launch: one per tile, at most about WGS_PER_CU per CU.
inline int stream_grid(int N) {
    const int NT = (N + 15) / 16;
    const int cap = device_cus() * SPECV_STREAM_WGS_PER_CU;
    return NT < cap ? NT : cap;
}

// Events for the next linear launch of this host thread (timing diagnostics).
static thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;

bool take_linear_timing(hipEvent_t* start, hipEvent_t* stop) {
    if (!g_time_start) return false;
    *start = g_time_start;
    *stop = g_time_stop;
    g_time_start = g_time_stop = nullptr;
    return true;
}

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

// A deeper load pipeline for matrices whose tiles give each CU at most one
// workgroup and whose waves walk many iterations (the long-K down projection
// of the 8B shape: K = 14336, 256 tiles): with four waves per CU, seven
// iterations in flight per wave hide more of the memory latency. Shapes with
// two workgroups per CU stream best with four (measured on MI355X: deeper
// pipelines there were slower). The depth must divide the iteration count,
// so no padding iterations are added.
constexpr int kDeepStages = 7;
inline bool deep_stream(int T, int N, int K) {
    const int J = (K / 32 + 15) / 16;
    const int NT = (N + 15) / 16;
    return J % kDeepStages == 0 && J >= 2 * kDeepStages && NT <= device_cus() &&
           stream_lds_bytes(T, K, false, false, kDeepStages) + (size_t)T * 512 <= kLdsBudget;
}

template <int T, bool AMAX, bool BS, bool RELOAD, int PROD = kProdNone, int P = SPECV_STREAM_STAGES>
static int launch_one(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                      Best* amax, int Tr, int N, int K, hipStream_t s, const ProdArgs& pa = ProdArgs{}) {
    static size_t lds_enabled = 64 * 1024;
    const size_t lds = stream_lds_bytes(T, K, BS, RELOAD, P) + prod_scratch_bytes(PROD, T, K);
    if (lds + (size_t)T * 512 > kLdsBudget) return SPECV_E_SHAPE;
    auto kernel = &w4a8_linear_stream_kernel<T, P, AMAX, BS, RELOAD, PROD>;
    const int rc = enable_lds(reinterpret_cast<const void*>(kernel), lds, lds_enabled);
    if (rc != SPECV_OK) return rc;
    const int grid = stream_grid(N);
    const int write_y = y != nullptr;
    if (g_time_start) {
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), lds, s, g_time_start, g_time_stop, 0, wq, ws, xq, N, K,
                              grid, Tr, xs, y, write_y, amax, pa);
        g_time_start = g_time_stop = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), lds, s, wq, ws, xq, N, K, grid, Tr, xs, y, write_y, amax,
                           pa);
    }
    return launch_status();
}

// A stage count that divides a tile's J iterations where the default would
// pad the tile with empty iterations (0: the default applies). Tiles shorter
// than the default pipeline (K <= 1536) take one stage per iteration, and
// those whose J is a multiple of 5 but not of 4 take 5. Measured on MI355X,
// per launch: the 896-input matrices of the 0.5B shape (J = 2) qkv 2.77 ->
// 2.36 us, gate_up 3.59 -> 3.22 us, lm_head at T = 8 31.1 -> 23.4 us; the
// 4864-input down projection (J = 10) 4.25 -> 3.61 us at T = 1 and 4.58 ->
// 4.40 us at T = 8 (two stages there: 5.00 us).
inline int exact_stages(int T, int K) {
    const int J = (K / 32 + 15) / 16;
    int P = 0;
    if (J < SPECV_STREAM_STAGES)
        P = J;
    else if (J % SPECV_STREAM_STAGES != 0 && J % 5 == 0)
        P = 5;
    if (P && stream_lds_bytes(T, K, false, false, P) + (size_t)T * 512 > kLdsBudget) P = 0;
    return P;
}

template <int T, bool AMAX, int PROD = kProdNone>
static int launch_exact(int P, const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                        Best* amax, int Tr, int N, int K, hipStream_t s, const ProdArgs& pa = ProdArgs{}) {
    switch (P) {
        case 1: return launch_one<T, AMAX, false, false, PROD, 1>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa);
        case 2: return launch_one<T, AMAX, false, false, PROD, 2>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa);
        case 3: return launch_one<T, AMAX, false, false, PROD, 3>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa);
        case 5: return launch_one<T, AMAX, false, false, PROD, 5>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa);
        default: return SPECV_E_SHAPE;
    }
}

template <int T, bool BS>
static int launch_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, Best* amax,
                    int Tr, int N, int K, hipStream_t s, const ProdArgs& pa) {
    const bool keep = stream_keeps(T, K, BS);
    if constexpr (T <= 16 && !BS) {
        if (deep_stream(T, N, K))
            return amax ? launch_one<T, true, false, false, kProdNone, kDeepStages>(wq, ws, xq, xs, y, amax, Tr, N,
                                                                                    K, s, pa)
                        : launch_one<T, false, false, false, kProdNone, kDeepStages>(wq, ws, xq, xs, y, nullptr, Tr,
                                                                                     N, K, s, pa);
        if (const int P = exact_stages(T, K))
            return amax ? launch_exact<T, true>(P, wq, ws, xq, xs, y, amax, Tr, N, K, s, pa)
                        : launch_exact<T, false>(P, wq, ws, xq, xs, y, nullptr, Tr, N, K, s, pa);
    }
    if constexpr (T <= 16 && !BS) {
        if (amax)
            return keep ? launch_one<T, true, false, false>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa)
                        : launch_one<T, true, false, true>(wq, ws, xq, xs, y, amax, Tr, N, K, s, pa);
    } else {
        if (amax) return SPECV_E_SHAPE;
    }
    return keep ? launch_one<T, false, BS, false>(wq, ws, xq, xs, y, nullptr, Tr, N, K, s, pa)
                : launch_one<T, false, BS, true>(wq, ws, xq, xs, y, nullptr, Tr, N, K, s, pa);
}

// Fused producers: T <= kNormMaxT (RMSNorm) or kRowsTokens (given rows),
// per-token scales, every iteration's activations and the producer's
// scratch kept in LDS.
bool linear_fused_supported(int prod, int T, int K) {
    if (T < 1 || T > 16 || K < 32 || K % 32 || (prod != kProdNorm && prod != kProdRows)) return false;
    if (prod == kProdRows && (K > 256 * 4 * kRowsRegs || T > kRowsTokens)) return false;
    if (prod == kProdNorm && T > kNormMaxT) return false;
    return stream_lds_bytes(T, K, false, false) + prod_scratch_bytes(prod, T, K) + (size_t)T * 512 <= kLdsBudget;
}

template <int T>
static int launch_fused(int prod, const ProdArgs& pa, const uint8_t* wq, const uint16_t* ws, float* y, Best* amax,
                        int N, int K, hipStream_t s) {
    if (const int P = exact_stages(T, K); P && stream_lds_bytes(T, K, false, false, P) +
                                                          prod_scratch_bytes(prod, T, K) + (size_t)T * 512 <= kLdsBudget) {
        if (prod == kProdNorm)
            return amax ? launch_exact<T, true, kProdNorm>(P, wq, ws, nullptr, nullptr, y, amax, T, N, K, s, pa)
                        : launch_exact<T, false, kProdNorm>(P, wq, ws, nullptr, nullptr, y, nullptr, T, N, K, s, pa);
        if (amax) return SPECV_E_SHAPE;
        return launch_exact<T, false, kProdRows>(P, wq, ws, nullptr, nullptr, y, nullptr, T, N, K, s, pa);
    }
    if (prod == kProdNorm)
        return amax ? launch_one<T, true, false, false, kProdNorm>(wq, ws, nullptr, nullptr, y, amax, T, N, K, s, pa)
                    : launch_one<T, false, false, false, kProdNorm>(wq, ws, nullptr, nullptr, y, nullptr, T, N, K, s,
                                                                     pa);
    if (amax) return SPECV_E_SHAPE;
    return launch_one<T, false, false, false, kProdRows>(wq, ws, nullptr, nullptr, y, nullptr, T, N, K, s, pa);
}

int linear_enqueue_fused(int prod, const ProdArgs& pa, const uint8_t* wq, const uint16_t* ws, float* y, Best* amax,
                         int T, int N, int K, hipStream_t s) {
    if (!linear_fused_supported(prod, T, K)) return SPECV_E_SHAPE;
    if (pa.epi != kEpiPlain && (amax || N % 16)) return SPECV_E_SHAPE;
    switch (T) {
#define SPECV_CASE(n) \
    case n: return launch_fused<n>(prod, pa, wq, ws, y, amax, N, K, s);
        SPECV_CASE(1) SPECV_CASE(2) SPECV_CASE(3) SPECV_CASE(4) SPECV_CASE(5) SPECV_CASE(6)
        SPECV_CASE(7) SPECV_CASE(8)
#undef SPECV_CASE
        default: return SPECV_E_SHAPE;
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

bool linear_argmax_supported(int T, int N, int K) { return T >= 1 && T <= 16 && N >= 1 && K >= 32; }

int linear_argmax_chunks(int T, int N, int K) { return linear_argmax_supported(T, N, K) ? stream_grid(N) : 0; }

// Validated arguments. y may be null when amax is set (T <= 16, per-token
// scales). bs: xs holds per-block scales [T][K/32]. pa.epi chooses what the
// linear writes (T <= 16).
static int linear_dispatch(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                           Best* amax, int T, int N, int K, bool bs, hipStream_t s,
                           const ProdArgs& pa = ProdArgs{}) {
    switch (T) {
#define SPECV_CASE(n)                                                      \
    case n:                                                                \
        return bs ? launch_T<n, true>(wq, ws, xq, xs, y, amax, n, N, K, s, pa) \
                  : launch_T<n, false>(wq, ws, xq, xs, y, amax, n, N, K, s, pa);
        SPECV_CASE(1) SPECV_CASE(2) SPECV_CASE(3) SPECV_CASE(4) SPECV_CASE(5) SPECV_CASE(6)
        SPECV_CASE(7) SPECV_CASE(8) SPECV_CASE(9) SPECV_CASE(10) SPECV_CASE(11) SPECV_CASE(12)
        SPECV_CASE(13) SPECV_CASE(14) SPECV_CASE(15) SPECV_CASE(16)
#undef SPECV_CASE
        default:
            if (T > 16 && T <= 32) {  // the 32-token bucket: dense products where they apply
                if (pa.epi != kEpiPlain) return SPECV_E_SHAPE;
                if (!bs && !amax && linear_dense_supported(T, K))
                    return linear_dense_enqueue(wq, ws, xq, xs, y, T, N, K, s);
                return bs ? launch_T<32, true>(wq, ws, xq, xs, y, amax, T, N, K, s, pa)
                          : launch_T<32, false>(wq, ws, xq, xs, y, amax, T, N, K, s, pa);
            }
            return SPECV_E_SHAPE;
    }
}

int linear_enqueue(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y, Best* amax,
                   int T, int N, int K, void* /*workspace*/, hipStream_t s, int epi) {
    if (epi != kEpiPlain && (amax || N % 16)) return SPECV_E_SHAPE;
    ProdArgs pa{};
    pa.epi = epi;
    return linear_dispatch(wq, ws, xq, xs, y, amax, T, N, K, false, s, pa);
}

// Shape and pointer checks shared by the linear entry points (N >= 1).
static int linear_args(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, int32_t T,
                       int32_t N, int32_t K) {
    if (T < 1 || T > 32 || N < 1 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32) return SPECV_E_SHAPE;
    if (packed_weight_bytes(N, K) >= (int64_t)1 << 31) return SPECV_E_SHAPE;
    if (!wq || !ws || !xq || !xs) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(ws, 2) || !aligned(xs, 4)) return SPECV_E_ALIGN;
    return SPECV_OK;
}

static bool empty_call(int32_t T, int32_t N, int32_t K) {
    return T >= 1 && T <= 32 && N == 0 && K >= 32 && K <= (1 << 20) && K % 32 == 0;
}

// Scratch of w4a8_linear_argmax_T_noalloc: the (value, lowest row) pair of
// every token and workgroup, T * chunks * 8 bytes (16 tokens x 1024
// workgroups at most). Each device holds its own copy until the process
// ends. Host code takes its device address from hipGetSymbolAddress, once per
// device, and passes that address to the kernels: the array's name itself is
// not a device address in host code.
constexpr size_t kNoAllocScratchBytes = 128 * 1024;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`.
static int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return SPECV_E_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return SPECV_E_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPECV_OK;
}

}  // namespace specv

extern "C" int specv_time_next_linear(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return SPECV_E_INVAL;
    specv::g_time_start = static_cast<hipEvent_t>(start_event);
    specv::g_time_stop = static_cast<hipEvent_t>(stop_event);
    return SPECV_OK;
}

extern "C" size_t w4a8_linear_workspace(int32_t, int32_t, int32_t) { return 0; }

extern "C" int w4a8_linear_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                             float* y, int32_t T, int32_t N, int32_t K, void* workspace,
                             size_t workspace_bytes, void* stream) {
    using namespace specv;
    (void)workspace;
    (void)workspace_bytes;
    if (empty_call(T, N, K)) return SPECV_OK;
    const int rc = linear_args(wq, ws, xq, xs, T, N, K);
    if (rc != SPECV_OK) return rc;
    if (!y) return SPECV_E_INVAL;
    if (!aligned(y, 4)) return SPECV_E_ALIGN;
    return linear_dispatch(wq, ws, xq, xs, y, nullptr, T, N, K, false, (hipStream_t)stream);
}

extern "C" int w4a8_linear_blocks_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs,
                                    float* y, int32_t T, int32_t N, int32_t K, void* stream) {
    using namespace specv;
    if (empty_call(T, N, K)) return SPECV_OK;
    const int rc = linear_args(wq, ws, xq, xs, T, N, K);
    if (rc != SPECV_OK) return rc;
    if (!y) return SPECV_E_INVAL;
    if (!aligned(y, 4)) return SPECV_E_ALIGN;
    return linear_dispatch(wq, ws, xq, xs, y, nullptr, T, N, K, true, (hipStream_t)stream);
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
    if (T < 1 || T > 16) return SPECV_E_SHAPE;
    const int rc = linear_args(wq, ws, xq, xs, T, N, K);
    if (rc != SPECV_OK) return rc;
    if (!argmax) return SPECV_E_INVAL;
    if (!aligned(y, 4) || !aligned(argmax, 4)) return SPECV_E_ALIGN;
    const size_t need = w4a8_linear_argmax_workspace(T, N, K);
    if (!workspace || workspace_bytes < need) return SPECV_E_WORKSPACE;
    if (!aligned(workspace, 8)) return SPECV_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    Best* part = static_cast<Best*>(workspace);
    const int lrc = linear_dispatch(wq, ws, xq, xs, y, part, T, N, K, false, s);
    if (lrc != SPECV_OK) return lrc;
    hipLaunchKernelGGL(argmax_finish_kernel, dim3(T), dim3(256), 0, s, part, linear_argmax_chunks(T, N, K), argmax);
    return launch_status();
}

extern "C" int w4a8_linear_argmax_T_noalloc(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                                            const float* xs, float* y, int32_t* argmax, int32_t T, int32_t N,
                                            int32_t K, void* stream) {
    using namespace specv;
    if (T < 1 || T > 16) return SPECV_E_SHAPE;
    const int rc = linear_args(wq, ws, xq, xs, T, N, K);
    if (rc != SPECV_OK) return rc;
    if (!argmax) return SPECV_E_INVAL;
    if (!aligned(y, 4) || !aligned(argmax, 4)) return SPECV_E_ALIGN;
    if (w4a8_linear_argmax_workspace(T, N, K) > kNoAllocScratchBytes) return SPECV_E_WORKSPACE;
    void* part = nullptr;
    const int src = scratch_address(&part);
    if (src != SPECV_OK) return src;
    hipStream_t s = (hipStream_t)stream;
    const int lrc = linear_dispatch(wq, ws, xq, xs, y, static_cast<Best*>(part), T, N, K, false, s);
    if (lrc != SPECV_OK) return lrc;
    hipLaunchKernelGGL(argmax_finish_kernel, dim3(T), dim3(256), 0, s, static_cast<const Best*>(part),
                       linear_argmax_chunks(T, N, K), argmax);
    return launch_status();
}
