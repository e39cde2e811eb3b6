// Per-token int8 activation quantisation (absmax scale, codes rounded to
// nearest-even). One workgroup per token: the absmax is a max, which is exact
// in any order, so the wave and workgroup reductions below need no fixed
// shape; the scale and reciprocal are single IEEE divisions.
#include "common.h"

namespace specv {

constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quantize_act_kernel(
    const float* __restrict__ x, int K, int8_t* __restrict__ xq, float* __restrict__ xs) {
    const int t = blockIdx.x;
    const float* row = x + (int64_t)t * K;
    int8_t* out = xq + (int64_t)t * K;

    float a = 0.0f;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) a = fmaxf(a, fabsf(row[k]));
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));

    __shared__ float wave_max[kQuantThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
    __syncthreads();
    a = wave_max[0];
    for (int w = 1; w < kQuantThreads / 64; w++) a = fmaxf(a, wave_max[w]);

    if (a == 0.0f) {
        if (threadIdx.x == 0) xs[t] = 0.0f;
        for (int k = threadIdx.x; k < K; k += kQuantThreads) out[k] = 0;
        return;
    }
    const QuantScale qs = quant_scale(a);
    if (threadIdx.x == 0) xs[t] = a / 127.0f;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) out[k] = (int8_t)(int)quant_code(row[k], qs);
}

// Register-resident variant for rows of up to 4*CH*256 values with K % 4 == 0
// and 16-byte aligned rows: every thread loads its CH float4 at once (one
// memory round trip), reduces the max, then quantises from registers and
// stores four codes per 32-bit word.
template <int CH>
__global__ __launch_bounds__(kQuantThreads) void quantize_act_reg_kernel(
    const float* __restrict__ x, int K, int8_t* __restrict__ xq, float* __restrict__ xs) {
    const int t = blockIdx.x;
    const int K4 = K >> 2;
    const auto rx = make_rsrc(x + (int64_t)t * K, (uint32_t)K * 4u);
    v4i raw[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const int i = c * kQuantThreads + threadIdx.x;
        raw[c] = load16(rx, ((uint32_t)i * 16u) | ((uint32_t)(i >= K4) << 31));
    }
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c++)
#pragma unroll
        for (int e = 0; e < 4; e++) a = fmaxf(a, fabsf(lane_f32(raw[c][e])));
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    __shared__ float wave_max[kQuantThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
    __syncthreads();
    a = wave_max[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; w++) a = fmaxf(a, wave_max[w]);

    const bool zero = (a == 0.0f);
    const QuantScale qs = quant_scale(a);
    if (threadIdx.x == 0) xs[t] = zero ? 0.0f : a / 127.0f;
    uint32_t* out = reinterpret_cast<uint32_t*>(xq + (int64_t)t * K);
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const int i = c * kQuantThreads + threadIdx.x;
        if (i < K4) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; e++)
                packed |= ((uint32_t)(int)quant_code(lane_f32(raw[c][e]), qs) & 0xffu) << (8 * e);
            out[i] = packed;
        }
    }
}

// Per-block variant (one scale per token and 32 inputs): eight lanes own a
// block, four values each; the block's max is taken over the eight lanes
// (exact in any order), and the scale and reciprocal are single IEEE
// divisions as above. Blocks are consecutive 128-byte runs of x, since
// K % 32 == 0, and xs[t][g] is the block's index in that run.
__global__ __launch_bounds__(kQuantThreads) void quantize_act_blocks_kernel(
    const float* __restrict__ x, int64_t nblocks, int8_t* __restrict__ xq, float* __restrict__ xs) {
    const int64_t gi = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const int64_t blk = gi >> 3;
    const int part = (int)(gi & 7);
    const bool ok = blk < nblocks;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (ok) v = *reinterpret_cast<const float4*>(x + 32 * blk + 4 * part);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    a = fmaxf(a, __shfl_xor(a, 4, 64));
    const bool zero = (a == 0.0f);
    const QuantScale qs = quant_scale(a);
    if (!ok) return;
    if (part == 0) xs[blk] = zero ? 0.0f : a / 127.0f;
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) packed |= ((uint32_t)(int)quant_code(e[i], qs) & 0xffu) << (8 * i);
    *reinterpret_cast<uint32_t*>(xq + 32 * blk + 4 * part) = packed;
}

}  // namespace specv

extern "C" int w4a8_quantize_act_blocks(const float* x, int32_t T, int32_t K, int8_t* xq, float* xs, void* stream) {
    using namespace specv;
    if (T < 0 || T > (1 << 20) || K < 32 || K > (1 << 24) || K % 32) return SPECV_E_SHAPE;
    if ((int64_t)T * K >= (int64_t)1 << 31) return SPECV_E_SHAPE;
    if (T == 0) return SPECV_OK;
    if (!x || !xq || !xs) return SPECV_E_INVAL;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xs, 4)) return SPECV_E_ALIGN;
    const int64_t nblocks = (int64_t)T * (K / 32);
    const int64_t grid = (nblocks * 8 + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(quantize_act_blocks_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, (hipStream_t)stream,
                       x, nblocks, xq, xs);
    return launch_status();
}

extern "C" int w4a8_quantize_act(const float* x, int32_t T, int32_t K, int8_t* xq, float* xs,
                                 void* stream) {
    using namespace specv;
    if (T < 0 || T > (1 << 20) || K < 1 || K > (1 << 24)) return SPECV_E_SHAPE;
    if (T == 0) return SPECV_OK;
    if (!x || !xq || !xs) return SPECV_E_INVAL;
    if (!aligned(x, 4) || !aligned(xs, 4)) return SPECV_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const int K4 = K / 4;
    const bool vec = K % 4 == 0 && aligned(x, 16) && aligned(xq, 4);
    if (vec && K4 <= 1 * kQuantThreads)
        hipLaunchKernelGGL(quantize_act_reg_kernel<1>, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    else if (vec && K4 <= 2 * kQuantThreads)
        hipLaunchKernelGGL(quantize_act_reg_kernel<2>, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    else if (vec && K4 <= 4 * kQuantThreads)
        hipLaunchKernelGGL(quantize_act_reg_kernel<4>, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    else if (vec && K4 <= 8 * kQuantThreads)
        hipLaunchKernelGGL(quantize_act_reg_kernel<8>, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    else if (vec && K4 <= 16 * kQuantThreads)
        hipLaunchKernelGGL(quantize_act_reg_kernel<16>, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    else
        hipLaunchKernelGGL(quantize_act_kernel, dim3(T), dim3(kQuantThreads), 0, s, x, K, xq, xs);
    return launch_status();
}
