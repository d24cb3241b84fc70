// Per-input-channel activation norms for Wanda scoring (zyxy.net Wanda lecture, section 2.1:
// the score of w_ij multiplies |w_ij| by the L2 norm of input channel j over the calibration tokens).
//
// HBM-bound stream: one wave per channel row of X (K x N bf16, row-major). Each lane issues 16-byte
// loads along N (4 in flight), squares in double, and the wave reduces with butterfly shuffles.
// Accumulating in double keeps the result within one fp32 rounding of the exact norm; the fp64 FMA
// rate is far above what the byte stream needs.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {

constexpr int kNormWaves = 4;  // rows per 256-thread workgroup

__global__ __launch_bounds__(256) void col_norms_kernel(const uint16_t* __restrict__ X, int64_t K, int64_t N,
                                                        int64_t ldx, float* __restrict__ norms, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (j >= K) return;  // whole wave
    const uint16_t* row = X + j * ldx;
    double s = 0.0;
    int64_t n_done = 0;
    if (vec) {
        // 16-byte chunks of 8 bf16; row start is 16-byte aligned (checked on the host)
        const int64_t nchunk = N >> 3;
        const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
        int64_t c = lane;
        for (; c + 192 < nchunk; c += 256) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) v[u] = __builtin_nontemporal_load(r4 + c + 64 * u);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    double a = (double)bf16_to_f32(w[h] & 0xFFFFu);
                    double b = (double)bf16_to_f32(w[h] >> 16);
                    s += a * a;
                    s += b * b;
                }
            }
        }
        for (; c < nchunk; c += 64) {
            u32x4 v = __builtin_nontemporal_load(r4 + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; h++) {
                double a = (double)bf16_to_f32(w[h] & 0xFFFFu);
                double b = (double)bf16_to_f32(w[h] >> 16);
                s += a * a;
                s += b * b;
            }
        }
        n_done = nchunk << 3;
    }
    for (int64_t n = n_done + lane; n < N; n += 64) {
        double a = (double)bf16_to_f32(row[n]);
        s += a * a;
    }
    s = wave_sum_f64(s);
    if (lane == 0) norms[j] = (float)__builtin_sqrt(s);
}

hipError_t launch_col_norms(const uint16_t* X, int64_t K, int64_t N, int64_t ldx, float* norms, hipStream_t s) {
    const int vec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);
    const int64_t blocks = (K + kNormWaves - 1) / kNormWaves;
    hipLaunchKernelGGL(col_norms_kernel, dim3((unsigned)blocks), dim3(256), 0, s, X, K, N, ldx, norms, vec);
    return hipGetLastError();
}

}  // namespace sp24
