// Shader-clock probe (measurement support): the rate of the sparse matrix instructions with nothing
// else in the way. Every wave issues 16 independent v_smfmac_f32_16x16x64_bf16 per iteration on
// register operands and records the shader-clock cycles (s_memtime) and 100 MHz real-time ticks
// (s_memrealtime) of its loop. 96 KB of dynamic LDS per workgroup keeps one workgroup (4 waves, one
// per SIMD) on each compute unit. The result is written, not the accumulators' values, so the loop is
// kept by an opaque use of the accumulators at the end.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace {

constexpr int NACC = 16;

__global__ __launch_bounds__(256) void sclk_probe_kernel(int iters, uint64_t* out) {
    extern __shared__ char lds_pad[];
    (void)lds_pad;
    f32x4 acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 ra;
    u32x8 rb;
#pragma unroll
    for (int i = 0; i < 4; i++) ra[i] = 0x3F803F80u ^ (threadIdx.x & 7);  // bf16 pairs near 1
#pragma unroll
    for (int i = 0; i < 8; i++) rb[i] = 0x3F803F80u ^ ((threadIdx.x + i) & 7);
    const bf16x8 a = __builtin_bit_cast(bf16x8, ra);
    const bf16x16 b = __builtin_bit_cast(bf16x16, rb);
    const int idx = 0x44444444;  // positions (0, 1) in every group
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int i = 0; i < NACC; i++) acc[i] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, acc[i], idx, 0, 0);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int i = 0; i < NACC; i++) asm volatile("" ::"v"(acc[i]));
    if ((threadIdx.x & 63) == 0) {
        const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
        out[2 * w] = c1 - c0;
        out[2 * w + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_sclk_probe(int64_t blocks, int iters, uint64_t* out, hipStream_t s) {
    hipLaunchKernelGGL(sclk_probe_kernel, dim3((unsigned)blocks), dim3(256), 96 * 1024, s, iters, out);
    return hipGetLastError();
}

}  // namespace sp24
