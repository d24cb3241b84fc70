// Measurement support: a plain streaming read, the achievable floor for a kernel that must read a given number
// of bytes once (launch ramp, tail and all). Every 16-byte word of the buffer is loaded once (non-temporal),
// and each workgroup writes the XOR of the words it read, so a test can check that all of them were read.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace {

constexpr int kThreads = 256, kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                               u32x4* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // kUnroll independent loads in flight per lane
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; u++) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    // XOR across the workgroup: lanes, then waves through LDS
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] ^= (uint32_t)__shfl_xor((int)acc[c], off, 64);
    __shared__ u32x4 part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        u32x4 w = part[0];
        for (int k = 1; k < kThreads / 64; k++) w ^= part[k];
        sink[blockIdx.x] = w;
    }
}

}  // namespace

int stream_read_blocks(int64_t bytes) {
    const int64_t n16 = bytes / 16;
    const int64_t want = (n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const int64_t cap = (int64_t)device_cus() * 8;  // eight workgroups per compute unit
    return (int)(want < 1 ? 1 : (want < cap ? want : cap));
}

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t s) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)stream_read_blocks(bytes)), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(src), bytes / 16, static_cast<u32x4*>(sink));
    return hipGetLastError();
}

}  // namespace sp24
