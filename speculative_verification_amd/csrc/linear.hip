// W4A8 linear for T = 1..16 tokens on CDNA4 matrix cores.
//
// Operation (GPU-Resident Speculative Decoding for In-Browser LLM Inference
// with WebGPU, Small-Batch Verification Kernels and Implementation):
//   d[t][n][g] = sum_{k in group g} q(n,k) * xq[t][k]   exact int32
//   p_g        = f32(scale[n][g]) * f32(d)               one rounding
//   y[t][n]    = xs[t] * R16(p_0 .. p_{G-1})             fixed order
// R16: slot s in 0..15 accumulates the groups g = s, s+16, s+32, ... in
// increasing g from +0, then slot s += slot s+off for off = 8, 4, 2, 1.
//
// Work decomposition. A workgroup owns 16 output rows and all K. Its four
// waves split the 16 R16 slots: wave w owns slots 4w..4w+3, so in iteration j
// it reads groups 16j+4w .. 16j+4w+3 of each row, 64 contiguous bytes per row
// (the four waves together stream 256 contiguous bytes per row per
// iteration). Lane l of a wave holds row l%16 and slot 4w + l/16, i.e. one
// 16-byte group of nibbles and its scale, and keeps that slot's running fp32
// sum for every token. The slot sums of the 16 slots meet in LDS at the end
// and combine in the R16 tree, then xs[t] scales the result.
//
// Integer dots. One v_mfma_i32_16x16x32_i8 computes, for 16 rows, the dots
// of one 8-input chunk of each of the wave's four groups against up to four
// tokens: B (32x16) carries the weights, lane quarter q supplying the chunk of
// slot 4w+q for row l%16; A (16x32) carries the activations block-diagonally,
// row m = 4h+t holding token t's chunk of slot 4w+h in k-quarter h and zeros
// elsewhere. Output element (m, n) = (4h+t, row) is then exactly the chunk
// dot of row n, slot 4w+h, token t, and it lands in lane 16h + n, register t:
// the lane that loaded that row's group and scale. Four chunks accumulate in
// the int32 accumulator, giving the exact group dot.
//
// Nibble decode. Codes are stored u = q + 8. Flipping bit 3 of each nibble
// gives the 4-bit two's complement of q; moving it into the high half of a
// byte gives the int8 value 16q. The dots therefore come out as 16d (exact,
// |16d| < 2^20), and the scale is pre-divided by 16 (exact: a power of two on
// a widened fp16 value), so f32(scale/16) * f32(16d) is the same real product
// as f32(scale) * f32(d) and rounds identically.
//
// Ragged shapes. All global loads go through buffer resources; a lane whose
// row or group is out of range, or whose activation row is a padding token,
// uses an out-of-range offset and receives zeros. A zero group contributes
// +0 to a slot, which never changes it (a slot is never -0).
#include "common.h"

namespace specv {

template <int T>
struct Stage {
    static constexpr int TT = (T + 3) / 4;
    v4i w;          // 16 bytes of nibbles: one group of one row
    uint16_t s;     // its fp16 scale
    v4i a[TT][2];   // 32 activation codes of one token per tile (or zeros)
};

__device__ __forceinline__ long mk64(int lo, int hi) {
    return (long)(((unsigned long)(unsigned)hi << 32) | (unsigned)lo);
}

template <int T, int P>
__global__ __launch_bounds__(256) void w4a8_linear_kernel(const uint8_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ ws,
                                                          const int8_t* __restrict__ xq,
                                                          const float* __restrict__ xs,
                                                          float* __restrict__ y, int N, int K) {
    constexpr int TT = (T + 3) / 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;        // output row within the block; MFMA column n
    const int q = lane >> 4;        // slot within the wave; k-quarter of B
    const int h = (lane & 15) >> 2; // slot of this lane's A row
    const int tp = lane & 3;        // token of this lane's A row within a tile
    const int row = blockIdx.x * 16 + r;
    const int G = K >> 5;
    const int J = (G + 15) >> 4;
    const int slot = 4 * wave + q;
    const bool row_ok = row < N;
    const bool a_active = (q == h);

    const auto rw = make_rsrc(wq, (uint32_t)((int64_t)N * (K / 2)));
    const auto rs = make_rsrc(ws, (uint32_t)((int64_t)N * G * 2));
    const auto rx = make_rsrc(xq, (uint32_t)(T * K));

    auto load_stage = [&](Stage<T>& st, int j) {
        const int g = 16 * j + slot;
        const bool ok = row_ok && g < G;
        st.w = load16(rw, ok ? (uint32_t)(row * (K / 2) + 16 * g) : kOOB);
        st.s = load2(rs, ok ? (uint32_t)((row * G + g) * 2) : kOOB);
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            const int t = 4 * tt + tp;
            const bool aok = a_active && t < T && g < G;
            const uint32_t off = aok ? (uint32_t)(t * K + 32 * g) : kOOB;
            st.a[tt][0] = load16(rx, off);
            st.a[tt][1] = load16(rx, off + 16u);
        }
    };

    float acc[T];
#pragma unroll
    for (int t = 0; t < T; t++) acc[t] = 0.0f;

    auto compute = [&](const Stage<T>& st) {
        long b[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const unsigned W = (unsigned)st.w[c] ^ 0x88888888u;
            const unsigned lo = (W << 4) & 0xF0F0F0F0u;  // even inputs, as 16q
            const unsigned hi = W & 0xF0F0F0F0u;         // odd inputs, as 16q
            const unsigned b0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            const unsigned b1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
            b[c] = mk64((int)b0, (int)b1);
        }
        v4i d[TT];
#pragma unroll
        for (int tt = 0; tt < TT; tt++) d[tt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                const v4i& a = st.a[tt][c >> 1];
                const long av = (c & 1) ? mk64(a[2], a[3]) : mk64(a[0], a[1]);
                d[tt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, b[c], d[tt], 0, 0, 0);
            }
        }
        const float s16 = (float)__builtin_bit_cast(_Float16, st.s) * 0.0625f;
#pragma unroll
        for (int tt = 0; tt < TT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                if (4 * tt + v < T) acc[4 * tt + v] = acc[4 * tt + v] + s16 * (float)d[tt][v];
    };

    Stage<T> st[P];
#pragma unroll
    for (int p = 0; p < P; p++)
        if (p < J) load_stage(st[p], p);
    for (int j0 = 0; j0 < J; j0 += P) {
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int j = j0 + p;
            if (j < J) {
                compute(st[p]);
                if (j + P < J) load_stage(st[p], j + P);
            }
        }
    }

    __shared__ float red[16][T][16];  // [slot][token][row]
#pragma unroll
    for (int t = 0; t < T; t++) red[slot][t][r] = acc[t];
    __syncthreads();
    if (threadIdx.x < 16 * T) {
        const int t = threadIdx.x >> 4;
        const int rr = threadIdx.x & 15;
        float a[16];
#pragma unroll
        for (int s = 0; s < 16; s++) a[s] = red[s][t][rr];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
            for (int s = 0; s < off; s++) a[s] = a[s] + a[s + off];
        const int orow = blockIdx.x * 16 + rr;
        if (orow < N) y[(int64_t)t * N + orow] = xs[t] * a[0];
    }
}

template <int T>
static void launch(const uint8_t* wq, const uint16_t* ws, const int8_t* xq, const float* xs, float* y,
                   int N, int K, hipStream_t s) {
    constexpr int P = 4;
    hipLaunchKernelGGL((w4a8_linear_kernel<T, P>), dim3((N + 15) / 16), dim3(256), 0, s, wq, ws, xq,
                       xs, y, N, K);
}

}  // namespace specv

extern "C" int w4a8_linear_T(const uint8_t* wq, const uint16_t* ws, const int8_t* xq,
                             const float* xs, float* y, int32_t T, int32_t N, int32_t K,
                             void* stream) {
    using namespace specv;
    if (T < 1 || T > 16 || N < 0 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32)
        return SPECV_E_SHAPE;
    if ((int64_t)N * (K / 2) >= (int64_t)1 << 31) return SPECV_E_SHAPE;
    if (N == 0) return SPECV_OK;
    if (!wq || !ws || !xq || !xs || !y) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(ws, 2) || !aligned(xs, 4) || !aligned(y, 4))
        return SPECV_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    switch (T) {
#define SPECV_CASE(n) \
    case n: launch<n>(wq, ws, xq, xs, y, N, K, s); break;
        SPECV_CASE(1) SPECV_CASE(2) SPECV_CASE(3) SPECV_CASE(4) SPECV_CASE(5) SPECV_CASE(6)
        SPECV_CASE(7) SPECV_CASE(8) SPECV_CASE(9) SPECV_CASE(10) SPECV_CASE(11) SPECV_CASE(12)
        SPECV_CASE(13) SPECV_CASE(14) SPECV_CASE(15) SPECV_CASE(16)
#undef SPECV_CASE
        default: return SPECV_E_SHAPE;
    }
    return launch_status();
}
