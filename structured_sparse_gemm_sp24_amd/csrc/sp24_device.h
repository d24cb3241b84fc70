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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// ---------------------------------------------------------------- register-only epilogue helpers
// An MFMA 16 x 16 accumulator fragment gives lane l = 16q + 4a + b rows 4q .. 4q+3 of column 4a + b;
// row-major outputs want runs along a row. quad_transpose: a 4 x 4 transpose inside each lane quad
// (b = 0..3) by two DPP exchanges -- with lane b ^ 2 (off-diagonal 2 x 2 blocks), then with lane b ^ 1
// -- leaves lane b with row 4q + b, columns 4a .. 4a+3.
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {  // value of lane b ^ 2 of the quad
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {  // value of lane b ^ 1 of the quad
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
}
// 32-bit elements: v[t] = row 4q + t of this lane's column on entry; on exit element t is column 4a + t
// of row 4q + b.
__device__ __forceinline__ void quad_transpose(uint32_t (&v)[4], int b) {
    const bool low = b < 2, even = (b & 1) == 0;
    const uint32_t r0 = dpp_xor2(low ? v[2] : v[0]), r1 = dpp_xor2(low ? v[3] : v[1]);
    const uint32_t x0 = low ? v[0] : r0, x1 = low ? v[1] : r1, x2 = low ? r0 : v[2], x3 = low ? r1 : v[3];
    const uint32_t s0 = dpp_xor1(even ? x1 : x0), s1 = dpp_xor1(even ? x3 : x2);
    v[0] = even ? x0 : s0;
    v[1] = even ? s0 : x1;
    v[2] = even ? x2 : s1;
    v[3] = even ? s1 : x3;
}
// fp32 rows -> bf16 (round to nearest even), then the same transpose on packed pairs: pack rows
// (0,1) and (2,3), swap packed words across b ^ 2, then 16-bit halves across b ^ 1 (one byte permute
// per word; `sel` is half_sel(b)). v[0] holds columns 4a, 4a+1 of row 4q + b on exit, v[1] columns
// 4a+2, 4a+3.
__device__ __forceinline__ uint32_t half_sel(int b) {
    // v_perm_b32 byte selectors over {hi = partner word, lo = own word}: even lanes keep their low half
    // and take the partner's low half as high half; odd lanes take the partner's high half as low half
    // and keep their high half
    return (b & 1) == 0 ? 0x05040100u : 0x03020706u;
}
__device__ __forceinline__ void quad_transpose_bf16(const float (&f)[4], uint32_t (&v)[2], int b, uint32_t sel) {
    const uint32_t p0 = pack_bf16x2_rne(f[0], f[1]);
    const uint32_t p1 = pack_bf16x2_rne(f[2], f[3]);
    const bool low = b < 2;
    const uint32_t r = dpp_xor2(low ? p1 : p0);
    const uint32_t x0 = low ? p0 : r, x1 = low ? r : p1;
    v[0] = __builtin_amdgcn_perm(dpp_xor1(x0), x0, sel);
    v[1] = __builtin_amdgcn_perm(dpp_xor1(x1), x1, sel);
}
// Quad transpose across four slots of W words: lane b of each quad takes slot f from lane f of its
// quad, so (lane b, slot f) -> (lane f, slot b). Used to give the 4 lanes of a quad 4 pieces of one
// output row: the memory pipeline merges a quad's stores into one request when they fall in one
// 128-byte line, and otherwise issues one per lane.
template <int W>
__device__ __forceinline__ void slot_transpose4(uint32_t (&v)[4][W], int b) {
#pragma unroll
    for (int w = 0; w < W; w++) {
        uint32_t u[4] = {v[0][w], v[1][w], v[2][w], v[3][w]};
        quad_transpose(u, b);
#pragma unroll
        for (int t = 0; t < 4; t++) v[t][w] = u[t];
    }
}

// ---------------------------------------------------------------- int8 GEMM epilogue
// GELU(y) = y Phi(y) = y/2 erfc(-y/sqrt 2) in fp32, from the rational approximation of Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26: for x >= 0, erfc(x) = e^{-x^2} sum_{i=1..5} a_i t^i with
// t = 1/(1 + p x), absolute error at most 1.5e-7. Two rewrites for fp32:
//  - the sum is expanded in s = 1 - t = p x t (coefficients below, exact binomial expansion), so the
//    hardware reciprocal's rounding error is not amplified where t is near 1;
//  - with r = erfc(|y|/sqrt 2)/2, GELU(y) = max(y, 0) - |y| r for either sign of y (y >= 0: y - y r;
//    y < 0: y r), one fused multiply-add and no branch or select.
// |error| <= 8 * 2^-24 * |y| against the exact GELU of the fp32 input (3.1 * 2^-24 * |y| in an fp32 emulation
// with the reciprocal and exp2 each off by one ulp either way).
namespace as7126 {
constexpr double P = 0.3275911;
constexpr double A[5] = {0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429};
constexpr double binom(int n, int k) {
    double c = 1.0;
    for (int j = 1; j <= k; j++) c = c * (n - k + j) / j;
    return c;
}
// half the coefficient of s^k in sum_i a_i (1 - s)^i
constexpr float half_b(int k) {
    double c = 0.0;
    for (int i = 1; i <= 5; i++)
        if (k <= i) c += A[i - 1] * binom(i, k) * ((k & 1) ? -1.0 : 1.0);
    return (float)(0.5 * c);
}
}  // namespace as7126

__device__ __forceinline__ float gelu_f32(float y) {
#pragma clang fp contract(off)
    constexpr float P = (float)(as7126::P * 0.70710678118654752);  // p / sqrt 2: t = 1 / (1 + p |y| / sqrt 2)
    constexpr float C = (float)(-0.5 * 1.4426950408889634);         // e^{-y^2/2} = 2^{C y^2}
    const float z = fabsf(y);
    const float pz = z * P;
    const float t = __builtin_amdgcn_rcpf(pz + 1.0f);
    const float s = pz * t;
    float q = as7126::half_b(5);
    q = fmaf(s, q, as7126::half_b(4));
    q = fmaf(s, q, as7126::half_b(3));
    q = fmaf(s, q, as7126::half_b(2));
    q = fmaf(s, q, as7126::half_b(1));
    q = fmaf(s, q, as7126::half_b(0));
    const float r = q * __builtin_amdgcn_exp2f((y * C) * y);  // erfc(|y| / sqrt 2) / 2
    return fmaf(-z, r, fmaxf(y, 0.0f));
}

__device__ __forceinline__ f32x4 gelu4_f32(f32x4 y) {
    return f32x4{gelu_f32(y[0]), gelu_f32(y[1]), gelu_f32(y[2]), gelu_f32(y[3])};
}

// The int8 GEMM's value pipeline for one accumulator of output row m: dequant (one rounding multiply),
// optional bias add (one rounding add), optional GELU.
__device__ __forceinline__ float i8_dequant(int acc, float sc, float bias, bool has_bias) {
#pragma clang fp contract(off)
    float y = __fmul_rn((float)acc, sc);
    if (has_bias) y = __fadd_rn(y, bias);
    return y;
}

__device__ __forceinline__ float i8_value(int acc, float sc, float bias, bool has_bias, bool gelu) {
    const float y = i8_dequant(acc, sc, bias, has_bias);
    return gelu ? gelu_f32(y) : y;
}

// Requantization to int8: clamp(rne(fl32(y * inv_scale)), -127, 127), as the low byte; inv_scale is
// fl32(1 / out_scale), computed once on the host. Computed as fl32(t + B) with B = 1.5 * 2^23, clamped to
// [B - 127, B + 127]: for |t| < 2^22 the sum lies in [2^23, 2^24), where the float spacing is 1, so the one
// rounding of the add is rne(t) (B is even, so ties go to the even code), and the code sits in the low
// mantissa bits as a two's complement byte; beyond that range the clamp decides either way. Three
// instructions and no conversion; the byte is taken straight from the float's bits.
__device__ __forceinline__ float quant_i8_biased(float y, float inv_scale) {
#pragma clang fp contract(off)
    constexpr float B = 12582912.0f;
    const float t = __fmul_rn(y, inv_scale);
    return __builtin_amdgcn_fmed3f(__fadd_rn(t, B), B - 127.0f, B + 127.0f);
}

__device__ __forceinline__ uint32_t quant_i8(float y, float inv_scale) {
    return __float_as_uint(quant_i8_biased(y, inv_scale)) & 0xFFu;
}

// Four codes packed into one word (element t in byte t): two byte permutes and an or.
__device__ __forceinline__ uint32_t quant_i8x4(const f32x4& y, float inv_scale) {
    const uint32_t q0 = __float_as_uint(quant_i8_biased(y[0], inv_scale));
    const uint32_t q1 = __float_as_uint(quant_i8_biased(y[1], inv_scale));
    const uint32_t q2 = __float_as_uint(quant_i8_biased(y[2], inv_scale));
    const uint32_t q3 = __float_as_uint(quant_i8_biased(y[3], inv_scale));
    // selector bytes 0-3 pick the second operand's bytes, 4-7 the first's, 0x0c gives zero
    return __builtin_amdgcn_perm(q1, q0, 0x0c0c0400u) | __builtin_amdgcn_perm(q3, q2, 0x04000c0cu);
}

// 4 x 4 byte transpose inside each lane quad: byte t of lane b's word (row t of column b) goes to byte b
// of lane t's word. Two exchanges: 16-bit halves with lane b ^ 2, then bytes with lane b ^ 1, each one
// DPP move and one byte permute.
__device__ __forceinline__ uint32_t quad_transpose_u8(uint32_t w, int b) {
    const uint32_t r = dpp_xor2(w);
    const uint32_t x = __builtin_amdgcn_perm(r, w, b < 2 ? 0x05040100u : 0x03020706u);
    const uint32_t s = dpp_xor1(x);
    return __builtin_amdgcn_perm(s, x, (b & 1) == 0 ? 0x06020400u : 0x03070105u);
}

// Wave-level sum of a double (64 lanes) by butterfly shuffles.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace sp24
