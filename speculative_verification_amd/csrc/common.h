// Internal helpers of libspecv: buffer resources with zero-filled
// out-of-range loads, launch checking, and the fp32 rules every kernel keeps.
//
// Every source of the library is compiled with -ffp-contract=off and without
// fast-math, so each fp32 expression below is one IEEE binary32 operation
// rounded to nearest-even, with denormals kept and correctly rounded division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specv.h"

namespace specv {

// A raw buffer resource over [base, base + bytes). Loads whose offset lies
// past `bytes` return zeros instead of touching memory, which lets the
// kernels fill ragged tiles without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // dword 3 = 0x00020000: 32-bit data format, as the CDNA3/CDNA4 ISA uses
    // for raw (untyped) buffer access.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Offset that is out of range for every buffer the library accepts (all are
// validated to be smaller than 2^31 bytes).
constexpr uint32_t kOOB = 0x80000000u;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint16_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// The same loads with the non-temporal cache policy (the `nt` bit), for data
// read once per pass, such as the weights of a linear: the caches need not
// keep them for a reuse that does not come.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ v4i load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT));
}
__device__ __forceinline__ uint16_t load2_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kCachePolicyNT);
}

// Agent-coherent cache policy (sc1) for data one workgroup publishes to
// another of the same launch: such stores and loads are coherent across the
// chip's separate L2 caches without whole-cache write-backs.
constexpr int kCachePolicySC1 = 16;

// (value, index) pair of an argmax reduction. "Better" is the larger value,
// or an equal value at a lower index: a total order on (value, -index) with
// -0 == +0, so every reduction shape yields the lowest index of the maximum.
struct Best {
    float v;
    int i;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Best of 16 aligned lanes (order-free), exchanged with DPP: quad permutes
// of lane ^ 1 and lane ^ 2, then the half-row and row mirrors.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
    const float ov = __builtin_bit_cast(float, dpp_i32<CTRL>(__builtin_bit_cast(int, v)));
    const int oi = dpp_i32<CTRL>(i);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}
__device__ __forceinline__ void best16(float& v, int& i) {
    best_step<0xB1>(v, i);
    best_step<0x4E>(v, i);
    best_step<0x141>(v, i);
    best_step<0x140>(v, i);
}

// Reinterpret one 32-bit lane of a loaded vector as fp32. The element is
// taken by value first: clang lowers __builtin_bit_cast applied directly to
// an ext-vector element expression as a cast of element 0.
__device__ __forceinline__ float lane_f32(int v) { return __builtin_bit_cast(float, v); }

// Deterministic exp: Cody-Waite reduction x = n*ln2 + r with ln2 split in
// C1 (9 significant bits, n*C1 exact for |n| <= 128) and C2 = fl(ln2 - C1),
// a degree-7 Taylor polynomial in r by Horner's rule (separate multiply and
// add), and 2^n assembled from its exponent bits.
__device__ __forceinline__ float det_exp(float x) {
    if (x > 88.0f) return __builtin_inff();
    if (x < -87.0f) return 0.0f;
    const float inv_ln2 = 0x1.715476p+0f;
    const float C1 = 0x1.63p-1f;
    const float C2 = -0x1.bd0106p-13f;
    const float n = __builtin_rintf(x * inv_ln2);
    const float r = (x - n * C1) - n * C2;
    float p = 0x1.a01a02p-13f;         // 1/7!
    p = p * r + 0x1.6c16c2p-10f;       // 1/6!
    p = p * r + 0x1.111112p-7f;        // 1/5!
    p = p * r + 0x1.555556p-5f;        // 1/4!
    p = p * r + 0x1.555556p-3f;        // 1/3!
    p = p * r + 0x1.0p-1f;             // 1/2!
    p = p * r + 1.0f;                  // 1/1!
    p = p * r + 1.0f;                  // 1/0!
    const int ni = (int)n;
    return p * __builtin_bit_cast(float, (uint32_t)(ni + 127) << 23);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + det_exp(-g)); }

// Per-token (or per-block) int8 quantisation with absmax a: scale a / 127,
// codes rint(x * 127 / a) clamped to +-127, nearest-even. Below 2^-64, x and
// a are first multiplied by 2^64 (exact), so 127 / a cannot overflow for a
// tiny but nonzero absmax; wherever 127 / a is finite the scaled form gives
// the bits of the plain one, since a power-of-two factor commutes with each
// rounding while the results stay normal. a == 0 gives inv = 0 (codes 0).
struct QuantScale {
    float pre, inv;
};
__device__ __forceinline__ QuantScale quant_scale(float a) {
    const float pre = a < 0x1p-64f ? 0x1p64f : 1.0f;
    return QuantScale{pre, a == 0.0f ? 0.0f : 127.0f / (a * pre)};
}
__device__ __forceinline__ float quant_code(float x, QuantScale s) {
    const float r = __builtin_rintf((x * s.pre) * s.inv);  // v_rndne_f32: nearest-even
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? SPECV_OK : SPECV_E_HIP;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes of a matrix of N rows and K inputs in the packed tile layout: rows
// padded to whole 16-row tiles, 16 bytes of nibbles and one fp16 scale per
// row and 32-input group.
__host__ __device__ inline int64_t packed_rows(int64_t N) { return (N + 15) / 16 * 16; }
__host__ __device__ inline int64_t packed_weight_bytes(int64_t N, int64_t K) { return packed_rows(N) * (K / 2); }
__host__ __device__ inline int64_t packed_scale_bytes(int64_t N, int64_t K) { return packed_rows(N) * (K / 32) * 2; }

}  // namespace specv
