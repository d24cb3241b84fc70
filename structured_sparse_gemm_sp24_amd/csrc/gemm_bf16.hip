// Sparse x dense GEMM, bf16 in, fp32 accumulate: Y = W_2:4 . X (NVIDIA blog on Ampere structured
// sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1 Step 3 -- the kept values meet only
// the activations their 2-bit positions select).
//
// On gfx950 that selection is done by v_smfmac_f32_16x16x64_bf16. Operand layout of one instruction
// (wave of 64 lanes, lane l = 16*q + r):
//   A (sparse, 16 x 64 dense): lane holds 8 kept values of row r covering dense columns
//       [16q, 16q+16) -- exactly 16 contiguous bytes of a row of `values`;
//   index: 16 bits per lane, 2 bits per kept value -- exactly 2 contiguous bytes of a row of `meta`;
//   B (dense, 64 x 16): lane holds column n = r, element e at row k = 8q + (e & 7) + 32 (e >> 3);
//   C/D (16 x 16 fp32): lane holds column r, rows 4q .. 4q+3.
// So the stored values + metadata feed the instruction with no repacking.
//
// The compressed weight is stored in that lane order (16-row x 64-column tiles, see include/sp24.h),
// so a wave's A operand is one contiguous 1 KB load and its index operand one 128 B load.
//
// This file holds the direct kernel: each wave owns a 16-row x (16*NF)-column tile, takes A and the
// index straight from global memory and gathers B element by element with bounds checks, through
// general element strides, so it works for every shape, layout (feature- or token-major), batch and
// row pitch. It serves the cases the others do not take: the few-token kernel (gemm_bf16_skinny.hip,
// N <= 64) and the LDS-tiled kernel (gemm_bf16_tiled.hip, N > 64), each within its alignment and
// size conditions.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {

// Element strides: X[k, n] at k * sxk + n * sxn, Y[m, n] at m * sym + n * syn; batch blockIdx.z adds
// z * sxb / z * syb.
struct DirectArgs {
    const uint16_t* vals;
    const uint8_t* meta;
    int64_t M, K, N;
    const uint16_t* X;
    int64_t sxk, sxn, sxb;
    void* Y;
    int64_t sym, syn, syb;
    int out_fp32;
};

template <int NF>
__global__ __launch_bounds__(256) void gemm_bf16_direct(DirectArgs d) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t m0 = ((int64_t)blockIdx.y * 4 + (threadIdx.x >> 6)) * 16;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NF;
    if (m0 >= d.M) return;  // whole wave
    const uint16_t* __restrict__ X = d.X + (int64_t)blockIdx.z * d.sxb;
    f32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // compressed tiles of this 16-row block: one 1 KB values tile and one 128 B metadata tile per 64
    // dense columns, already in lane order (rows and columns are padded, so every tile exists)
    const int64_t tiles_per_row = (d.K + 63) / 64;
    const u32x4* vt = reinterpret_cast<const u32x4*>(d.vals) + (m0 >> 4) * tiles_per_row * 64 + lane;
    const uint16_t* mt = reinterpret_cast<const uint16_t*>(d.meta) + (m0 >> 4) * tiles_per_row * 64 + lane;
    for (int64_t t = 0; t < tiles_per_row; t++) {
        const int64_t k0 = 64 * t;
        const u32x4 a = vt[64 * t];
        const uint32_t idx = mt[64 * t];
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int64_t n = n0 + 16 * f + r;
            uint32_t b[8];
#pragma unroll
            for (int h = 0; h < 8; h++) {
                uint32_t v2 = 0;
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    const int e = 2 * h + s;
                    const int64_t k = k0 + 8 * q + (e & 7) + 32 * (e >> 3);
                    uint32_t v = 0;
                    if (n < d.N && k < d.K) v = X[k * d.sxk + n * d.sxn];
                    v2 |= v << (16 * s);
                }
                b[h] = v2;
            }
            const u32x8 bv = {b[0], b[1], b[2], b[3], b[4], b[5], b[6], b[7]};
            acc[f] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                               __builtin_bit_cast(bf16x16, bv), acc[f], (int)idx, 0, 0);
        }
    }
    char* const Y = static_cast<char*>(d.Y) + (int64_t)blockIdx.z * d.syb * (d.out_fp32 ? 4 : 2);
#pragma unroll
    for (int f = 0; f < NF; f++) {
        const int64_t n = n0 + 16 * f + r;
        if (n >= d.N) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t m = m0 + 4 * q + i;
            if (m >= d.M) continue;
            const int64_t o = m * d.sym + n * d.syn;
            if (d.out_fp32)
                reinterpret_cast<float*>(Y)[o] = acc[f][i];
            else
                reinterpret_cast<uint16_t*>(Y)[o] = f32_to_bf16_rne(acc[f][i]);
        }
    }
}

static hipError_t launch_gemm_bf16_direct(const GemmArgs& g, hipStream_t s) {
    DirectArgs d;
    d.vals = static_cast<const uint16_t*>(g.values);
    d.meta = g.meta;
    d.M = g.M; d.K = g.K; d.N = g.N;
    d.X = static_cast<const uint16_t*>(g.X);
    d.sxk = g.tm ? 1 : g.ldx;
    d.sxn = g.tm ? g.ldx : 1;
    d.sxb = g.sx;
    d.Y = g.Y;
    d.sym = g.tm ? 1 : g.ldy;
    d.syn = g.tm ? g.ldy : 1;
    d.syb = g.sy;
    d.out_fp32 = g.out_fp32;
    const unsigned gy = (unsigned)((g.M + 63) / 64);
    // grid z covers at most 65535 batch entries per launch
    for (int64_t b0 = 0; b0 < g.batch; b0 += 65535) {
        const unsigned gz = (unsigned)(g.batch - b0 < 65535 ? g.batch - b0 : 65535);
        DirectArgs e = d;
        e.X = d.X + b0 * d.sxb;
        e.Y = static_cast<char*>(d.Y) + b0 * d.syb * (g.out_fp32 ? 4 : 2);
        if (g.N <= 16)
            hipLaunchKernelGGL(gemm_bf16_direct<1>, dim3((unsigned)((g.N + 15) / 16), gy, gz), dim3(256), 0, s, e);
        else
            hipLaunchKernelGGL(gemm_bf16_direct<4>, dim3((unsigned)((g.N + 63) / 64), gy, gz), dim3(256), 0, s, e);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
    if (gemm_bf16_fewtok_ok(g)) return launch_gemm_bf16_fewtok(g, s);
    if (gemm_bf16_skinny_ok(g)) return launch_gemm_bf16_skinny(g, s);
    if (gemm_bf16_tiled_ok(g)) return launch_gemm_bf16_tiled(g, s);
    return launch_gemm_bf16_direct(g, s);
}

}  // namespace sp24
