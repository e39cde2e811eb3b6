// Measurement diagnostics (not part of the computation): a plain streaming
// read, so a benchmark can put the linear kernels next to the rate the same
// bytes stream at with no arithmetic, and an empty launch (zero bytes) for
// the per-launch cost of the queue.
#include "common.h"

namespace specv {

// Each thread reads 16 bytes per step with four loads in flight, striding
// by the whole grid; the folded value is stored only if it equals a
// sentinel, which keeps the loads without writing anything in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const int4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const int4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (uint32_t)(a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const int4 a = p[i];
        acc ^= (uint32_t)(a.x ^ a.y ^ a.z ^ a.w);
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace specv

extern "C" int specv_stream_read(const void* p, size_t bytes, uint32_t* sink, int32_t grid, void* stream) {
    using namespace specv;
    if (grid < 1 || grid > 65536 || bytes % 16 || (bytes && !p) || !sink) return SPECV_E_INVAL;
    if (!aligned(p, 16) || !aligned(sink, 4)) return SPECV_E_ALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const int4*>(p), bytes / 16, sink);
    return launch_status();
}
