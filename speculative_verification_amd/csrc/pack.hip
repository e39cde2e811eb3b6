// Packed tile layout of the W4A8 weights.
//
// The interchange format is [P2]'s (WebGPU for LLM Inference, A quantised
// matrix-vector kernel in WGSL): nibbles row-major, two inputs per byte, one
// fp16 scale per row and 32-input group. The linear kernels walk 16-row
// tiles group by group, so the packed layout stores a tile's 16-byte group
// chunks in that order: chunk c = (t * G + g) * 16 + r holds row 16t + r,
// group g. A wavefront's load of four groups of a tile is then one
// contiguous kilobyte, and a workgroup's tile one contiguous stream. Scales
// follow the same chunk order, one fp16 value per chunk. Rows past N (the
// padding of the last tile) are zero.
#include "common.h"

namespace specv {

__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ wq,
                                                           const uint16_t* __restrict__ ws, int N, int K,
                                                           uint8_t* __restrict__ wp, uint16_t* __restrict__ sp,
                                                           int64_t chunks) {
    const int64_t G = K >> 5;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
        const int64_t r = c & 15, tg = c >> 4;
        const int64_t t = tg / G, g = tg - t * G;
        const int64_t row = 16 * t + r;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        uint16_t sc = 0;
        if (row < N) {
            v = *reinterpret_cast<const uint4*>(wq + row * (K / 2) + 16 * g);
            sc = ws[row * G + g];
        }
        *reinterpret_cast<uint4*>(wp + c * 16) = v;
        sp[c] = sc;
    }
}

static bool pack_shape_ok(int32_t N, int32_t K) {
    if (N < 1 || N > (1 << 24) || K < 32 || K > (1 << 20) || K % 32) return false;
    return packed_weight_bytes(N, K) < ((int64_t)1 << 31);
}

}  // namespace specv

extern "C" size_t w4a8_packed_weight_bytes(int32_t N, int32_t K) {
    return specv::pack_shape_ok(N, K) ? (size_t)specv::packed_weight_bytes(N, K) : 0;
}

extern "C" size_t w4a8_packed_scale_bytes(int32_t N, int32_t K) {
    return specv::pack_shape_ok(N, K) ? (size_t)specv::packed_scale_bytes(N, K) : 0;
}

extern "C" int w4a8_pack_weights(const uint8_t* wq, const uint16_t* ws, int32_t N, int32_t K, uint8_t* wp,
                                 uint16_t* sp, void* stream) {
    using namespace specv;
    if (!pack_shape_ok(N, K)) return SPECV_E_SHAPE;
    if (!wq || !ws || !wp || !sp) return SPECV_E_INVAL;
    if (!aligned(wq, 16) || !aligned(wp, 16) || !aligned(ws, 2) || !aligned(sp, 2)) return SPECV_E_ALIGN;
    const int64_t chunks = packed_scale_bytes(N, K) / 2;
    const int64_t blocks = (chunks + 255) / 256;
    const int grid = (int)(blocks < 8192 ? blocks : 8192);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, wq, ws, N, K, wp, sp,
                       chunks);
    return launch_status();
}
