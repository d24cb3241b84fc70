// Sparse x dense GEMM in int8 with exact int32 accumulation and a per-output-channel dequant
// epilogue (oeforum post on sparse acceleration: int8 and 2:4 combine; Orin NN design, Chapter 7,
// section 3.1 Step 4, sparse + INT8).
//
// gfx950's v_smfmac_i32_16x16x128_i8 operand layout (lane l = 16*q + r):
//   A (sparse, 16 x 128 dense): lane holds 16 kept int8 of row r covering dense columns
//       [32q, 32q+32) -- 16 contiguous bytes of a row of `values`;
//   index: 32 bits per lane (8 groups) -- 4 contiguous bytes of a row of `meta`;
//   B (dense, 128 x 16): lane holds column r, element e at row k = 16q + (e & 15) + 64 (e >> 4);
//   C/D (16 x 16 int32): lane holds column r, rows 4q .. 4q+3.
// Epilogue: y = fl32( fl32(acc) * scale[m] ), a single rounding multiply; optionally + bias[m] (one rounding
// add) and GELU, stored as fp32, bf16 (round to nearest even) or int8 codes clamp(rne(y * inv_scale)).
//
// The compressed weight is stored in that lane order (16-row x 128-column tiles, see include/sp24.h).
// Direct kernel: each wave owns a 16 x (16*NF) tile, reads A (1 KB) and the index (256 B) of each
// tile from global memory and gathers B element by element with bounds checks through general element
// strides (any shape, layout, batch and row pitch). The LDS-tiled kernel (gemm_i8_tiled.hip) takes
// over for N > 64 with 16-byte X rows.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {

// Element strides: X[k, n] at k * sxk + n * sxn, Y[m, n] at m * sym + n * syn; batch blockIdx.z adds
// z * sxb / z * syb.
struct DirectArgsI8 {
    const int8_t* vals;
    const uint8_t* meta;
    int64_t M, K, N;
    const int8_t* X;
    int64_t sxk, sxn, sxb;
    const float* scale;
    const float* bias;
    int gelu, out_kind;
    float inv_scale;
    void* Y;
    int64_t sym, syn, syb;
};

template <int NF>
__global__ __launch_bounds__(256) void gemm_i8_direct(DirectArgsI8 d) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t m0 = ((int64_t)blockIdx.y * 4 + (threadIdx.x >> 6)) * 16;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NF;
    if (m0 >= d.M) return;  // whole wave
    const int8_t* __restrict__ X = d.X + (int64_t)blockIdx.z * d.sxb;
    i32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) acc[f] = i32x4{0, 0, 0, 0};

    // compressed tiles of this 16-row block: 1 KB of values and 256 B of metadata per 128 dense
    // columns, in lane order (padded rows/columns hold zeros and canonical metadata)
    const int64_t tiles_per_row = (d.K + 127) / 128;
    const u32x4* vt = reinterpret_cast<const u32x4*>(d.vals) + (m0 >> 4) * tiles_per_row * 64 + lane;
    const uint32_t* mt = reinterpret_cast<const uint32_t*>(d.meta) + (m0 >> 4) * tiles_per_row * 64 + lane;
    for (int64_t t = 0; t < tiles_per_row; t++) {
        const int64_t k0 = 128 * t;
        const u32x4 a = vt[64 * t];
        const uint32_t idx = mt[64 * t];
        const i32x4 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int64_t n = n0 + 16 * f + r;
            uint32_t b[8];
#pragma unroll
            for (int w = 0; w < 8; w++) {
                uint32_t v4 = 0;
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    const int e = 4 * w + s;
                    const int64_t k = k0 + 16 * q + (e & 15) + 64 * (e >> 4);
                    uint32_t v = 0;
                    if (n < d.N && k < d.K) v = (uint8_t)X[k * d.sxk + n * d.sxn];
                    v4 |= v << (8 * s);
                }
                b[w] = v4;
            }
            const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
            acc[f] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, acc[f], (int)idx, 0, 0);
        }
    }
    const int es = d.out_kind == OUT_BF16 ? 2 : (d.out_kind == OUT_I8 ? 1 : 4);
    char* const Y = static_cast<char*>(d.Y) + (int64_t)blockIdx.z * d.syb * es;
#pragma unroll
    for (int f = 0; f < NF; f++) {
        const int64_t n = n0 + 16 * f + r;
        if (n >= d.N) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t m = m0 + 4 * q + i;
            if (m >= d.M) continue;
            const int64_t o = m * d.sym + n * d.syn;
            if (d.out_kind == OUT_I32) {
                reinterpret_cast<int32_t*>(Y)[o] = acc[f][i];
                continue;
            }
            const float y = i8_value(acc[f][i], d.scale[m], d.bias ? d.bias[m] : 0.f, d.bias != nullptr, d.gelu != 0);
            if (d.out_kind == OUT_F32)
                reinterpret_cast<float*>(Y)[o] = y;
            else if (d.out_kind == OUT_BF16)
                reinterpret_cast<uint16_t*>(Y)[o] = f32_to_bf16_rne(y);
            else
                reinterpret_cast<uint8_t*>(Y)[o] = (uint8_t)quant_i8(y, d.inv_scale);
        }
    }
}

hipError_t launch_gemm_i8(const GemmArgs& g, hipStream_t s) {
    if (gemm_i8_fewtok_ok(g)) return launch_gemm_i8_fewtok(g, s);
    if (gemm_i8_tiled_ok(g)) return launch_gemm_i8_tiled(g, s);
    DirectArgsI8 d;
    d.vals = static_cast<const int8_t*>(g.values);
    d.meta = g.meta;
    d.M = g.M; d.K = g.K; d.N = g.N;
    d.X = static_cast<const int8_t*>(g.X);
    d.sxk = g.tm ? 1 : g.ldx;
    d.sxn = g.tm ? g.ldx : 1;
    d.sxb = g.sx;
    d.scale = g.scale;
    d.bias = g.bias;
    d.gelu = g.gelu;
    d.out_kind = g.out_kind;
    d.inv_scale = g.inv_scale;
    d.Y = g.Y;
    d.sym = g.tm ? 1 : g.ldy;
    d.syn = g.tm ? g.ldy : 1;
    d.syb = g.sy;
    const unsigned gy = (unsigned)((g.M + 63) / 64);
    // grid z covers at most 65535 batch entries per launch
    for (int64_t b0 = 0; b0 < g.batch; b0 += 65535) {
        const unsigned gz = (unsigned)(g.batch - b0 < 65535 ? g.batch - b0 : 65535);
        DirectArgsI8 e = d;
        e.X = d.X + b0 * d.sxb;
        e.Y = static_cast<char*>(d.Y) + b0 * d.syb * (g.out_kind == OUT_BF16 ? 2 : (g.out_kind == OUT_I8 ? 1 : 4));
        if (g.N <= 16)
            hipLaunchKernelGGL(gemm_i8_direct<1>, dim3((unsigned)((g.N + 15) / 16), gy, gz), dim3(256), 0, s, e);
        else
            hipLaunchKernelGGL(gemm_i8_direct<4>, dim3((unsigned)((g.N + 63) / 64), gy, gz), dim3(256), 0, s, e);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace sp24
