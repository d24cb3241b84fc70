// Device-side types and helpers shared by the sp24 HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sp24 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// fp32 -> bf16 bits, round to nearest even (adding 0x7FFF plus the kept lsb carries exactly at and
// above the halfway point; overflow to infinity comes out right). NaN becomes a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32. Same
// result as f32_to_bf16_rne for every finite value and infinities (NaN payloads may differ).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// IEEE half bits -> float (exact).
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

// Compressed layout: byte b of compressed row i, for tiles of T bytes per row (T = 64 for values,
// KT/8 for metadata, KT = 128 / value size), 16-row tiles stored row block by row block and along K
// inside a block, each row's tile bytes cut into 4 quarters stored quarter-major.
template <int T>
__device__ __forceinline__ int64_t tiled_offset(int64_t i, int64_t b, int64_t tiles_per_row) {
    constexpr int Q = T / 4;
    const int64_t t = b / T;
    const int rem = (int)(b - t * T);
    return (((i >> 4) * tiles_per_row + t) * 4 + rem / Q) * (16 * Q) + (i & 15) * Q + rem % Q;
}

// Wave-level sum of a double (64 lanes) by butterfly shuffles.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace sp24
