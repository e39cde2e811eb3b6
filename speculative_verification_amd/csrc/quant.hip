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
    const float inv = 127.0f / a;
    if (threadIdx.x == 0) xs[t] = a / 127.0f;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) {
        float r = __builtin_rintf(row[k] * inv);  // v_rndne_f32: nearest-even
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        out[k] = (int8_t)(int)r;
    }
}

}  // namespace specv

extern "C" int w4a8_quantize_act(const float* x, int32_t T, int32_t K, int8_t* xq, float* xs,
                                 void* stream) {
    using namespace specv;
    if (T < 0 || T > 64 || K < 1 || K > (1 << 24)) return SPECV_E_SHAPE;
    if (T == 0) return SPECV_OK;
    if (!x || !xq || !xs) return SPECV_E_INVAL;
    if (!aligned(x, 4) || !aligned(xs, 4)) return SPECV_E_ALIGN;
    hipLaunchKernelGGL(quantize_act_kernel, dim3(T), dim3(kQuantThreads), 0, (hipStream_t)stream,
                       x, K, xq, xs);
    return launch_status();
}
