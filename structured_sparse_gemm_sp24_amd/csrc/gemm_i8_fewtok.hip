// Sparse x dense int8 GEMM for a few tokens in the Linear layout (token-major X, N <= 64), exact int32
// accumulation, the optional per-output-channel fp32 dequant and the fused FFN epilogue (bias, GELU, bf16
// or requantized int8 output) (oeforum post on sparse acceleration: int8 and 2:4 combine; NVIDIA blog on
// Ampere structured sparsity, Figure 1 and its quantization section; Orin NN design, Chapter 7, section
// 3.1 Step 4).
//
// With N this small the product streams the compressed int8 weight (0.625 bytes per dense weight) from
// HBM once, and X (N rows of K bytes) stays in L2. A workgroup owns R consecutive 16-row blocks and all N
// tokens (NF fragments of 16); its S waves split the K tiles (128 dense columns each) into contiguous
// ranges. A wave requests U tiles' operands at a time before their smfmacs:
//  - per lane and block, the 16-byte run of its slot in the compressed value tile and its 32-bit index
//    (both already in v_smfmac_i32_16x16x128_i8 operand order);
//  - per fragment, two 16-byte runs of its token's row, k0 + 16q .. +15 and k0 + 64 + 16q .. +15 (the
//    B operand's two halves, lane = token).
// Every read goes through a buffer descriptor: blocks past M, tokens past N and the tiles past a wave's
// range read zeros, and nothing else is read. The waves' int32 partial sums are added through LDS (exact
// in any order), then wave 0 runs the epilogue value pipeline of the tiled int8 kernel on each accumulator
// (y = fl32(fl32(acc) * scale[m]), then fl32(y + bias[m]), then GELU, then the output conversion; each step
// one rounding) and stores, per lane, four consecutive output channels of one token.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace fewtok_i8 {

constexpr int KT = 128;  // dense K per compressed tile
constexpr uint32_t OOR = 0x80000000u;  // a byte offset past every record count: the load returns zeros

struct Args {
    const int8_t* vals;
    const uint8_t* meta;
    const int8_t* X;
    const float* scale;
    const float* bias;
    float inv_scale;  // int8 output: fl32(1 / out_scale)
    void* Y;
    int64_t M, K, N, ldx, sxb, ldy, syb;
    int y_vec;  // 16-byte output stores allowed (aligned Y, row pitch and batch stride multiples of 4)
};

// Raw buffer descriptor over `bytes` bytes (every extent here is a multiple of 16).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// OUT: OUT_I32 (raw accumulators), OUT_F32, OUT_BF16, OUT_I8; EPI: bias (1) | GELU (2).
template <int NF, int R, int U, int S, int OUT, int EPI>
__global__ __launch_bounds__(64 * S) void gemm_i8_fewtok_kernel(Args a) {
    __shared__ i32x4 red[(S - 1) * R * NF * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int64_t nb = (a.M + 15) / 16, b0 = (int64_t)blockIdx.x * R;
    const int T = (int)(a.K / KT);
    const int64_t blocks = nb - b0 < R ? nb - b0 : R;
    const __amdgpu_buffer_rsrc_t rA = rsrc(a.vals + b0 * T * 1024, blocks * T * 1024);
    const __amdgpu_buffer_rsrc_t rM = rsrc(a.meta + b0 * T * 256, blocks * T * 256);
    const int8_t* X = a.X + (int64_t)blockIdx.y * a.sxb;
    const __amdgpu_buffer_rsrc_t rX = rsrc(X, (a.N - 1) * a.ldx + a.K);
    uint32_t xo[NF];  // this lane's token row (+16q), or past the descriptor for tokens past N
#pragma unroll
    for (int f = 0; f < NF; f++) {
        const int64_t n = 16 * f + r;
        xo[f] = n < a.N ? (uint32_t)(n * a.ldx + 16 * q) : OOR;
    }
    const int per = (T + S - 1) / S, t0 = wave * per, t1 = t0 + per < T ? t0 + per : T;

    i32x4 acc[R][NF];
#pragma unroll
    for (int i = 0; i < R; i++)
#pragma unroll
        for (int f = 0; f < NF; f++) acc[i][f] = i32x4{0, 0, 0, 0};

#pragma unroll 1
    for (int t = t0; t < t1; t += U) {
        i32x4 av[U][R];
        int iv[U][R];
        i32x8 bv[U][NF];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const bool in = t + u < t1;  // tiles past the range read zeros (and add nothing)
#pragma unroll
            for (int i = 0; i < R; i++) {
                const uint32_t ta = in ? (uint32_t)((i * T + t + u) * 1024 + 16 * lane) : OOR;
                const uint32_t tm = in ? (uint32_t)((i * T + t + u) * 256 + 4 * lane) : OOR;
                av[u][i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, (int)ta, 0, 0));
                iv[u][i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rM, (int)tm, 0, 0);
            }
#pragma unroll
            for (int f = 0; f < NF; f++) {
                const uint32_t o = in ? xo[f] + (uint32_t)((t + u) * KT) : OOR;
                const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, (int)o, 0, 0));
                const i32x4 hi =
                    __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, (int)(o + 64u), 0, 0));
                bv[u][f] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int i = 0; i < R; i++)
#pragma unroll
                for (int f = 0; f < NF; f++)
                    acc[i][f] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[u][i], bv[u][f], acc[i][f], iv[u][i], 0, 0);
    }

    // partial sums of waves 1 .. S-1 through LDS; wave 0 adds them (integer adds: any order is exact)
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < R; i++)
#pragma unroll
            for (int f = 0; f < NF; f++) red[(((wave - 1) * R + i) * NF + f) * 64 + lane] = acc[i][f];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll 1
    for (int w = 1; w < S; w++)
#pragma unroll
        for (int i = 0; i < R; i++)
#pragma unroll
            for (int f = 0; f < NF; f++) acc[i][f] += red[(((w - 1) * R + i) * NF + f) * 64 + lane];

    // lane (q, r): output channels 16 b + 4q .. +3 of token 16 f + r (the accumulator's four rows)
    constexpr int ES = OUT == OUT_BF16 ? 2 : (OUT == OUT_I8 ? 1 : 4);
    constexpr bool BIAS = (EPI & 1) != 0, GELU = (EPI & 2) != 0;
    char* const Y = static_cast<char*>(a.Y) + (int64_t)blockIdx.y * a.syb * ES;
#pragma unroll
    for (int i = 0; i < R; i++) {
        const int64_t m0 = 16 * (b0 + i) + 4 * q;
        if (m0 >= a.M) continue;
        float sc[4] = {1.f, 1.f, 1.f, 1.f}, bi[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if constexpr (OUT != OUT_I32) sc[j] = m0 + j < a.M ? a.scale[m0 + j] : 0.f;
            if constexpr (BIAS) bi[j] = m0 + j < a.M ? a.bias[m0 + j] : 0.f;
        }
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int64_t n = 16 * f + r;
            if (n >= a.N) continue;
            uint32_t e[4];  // the four output elements' bits
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if constexpr (OUT == OUT_I32) {
                    e[j] = (uint32_t)acc[i][f][j];
                } else {
                    const float y = i8_value(acc[i][f][j], sc[j], bi[j], BIAS, GELU);
                    if constexpr (OUT == OUT_F32) e[j] = __float_as_uint(y);
                    else if constexpr (OUT == OUT_BF16) e[j] = f32_to_bf16_rne(y);
                    else e[j] = quant_i8(y, a.inv_scale);
                }
            }
            char* const p = Y + (n * a.ldy + m0) * ES;
            if (a.y_vec && m0 + 3 < a.M) {
                if constexpr (ES == 4) *reinterpret_cast<u32x4*>(p) = u32x4{e[0], e[1], e[2], e[3]};
                else if constexpr (ES == 2) *reinterpret_cast<u32x2*>(p) = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                else *reinterpret_cast<uint32_t*>(p) = e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24);
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if (m0 + j >= a.M) continue;
                    if constexpr (ES == 4) reinterpret_cast<uint32_t*>(p)[j] = e[j];
                    else if constexpr (ES == 2) reinterpret_cast<uint16_t*>(p)[j] = (uint16_t)e[j];
                    else reinterpret_cast<uint8_t*>(p)[j] = (uint8_t)e[j];
                }
            }
        }
    }
}

template <int NF, int R, int U, int S, int OUT>
static void launch_epi(int epi, dim3 grd, dim3 blk, hipStream_t s, const Args& e) {
    switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_i8_fewtok_kernel<NF, R, U, S, OUT, 0>), grd, blk, 0, s, e); break;
    case 1: hipLaunchKernelGGL((gemm_i8_fewtok_kernel<NF, R, U, S, OUT, 1>), grd, blk, 0, s, e); break;
    case 2: hipLaunchKernelGGL((gemm_i8_fewtok_kernel<NF, R, U, S, OUT, 2>), grd, blk, 0, s, e); break;
    default: hipLaunchKernelGGL((gemm_i8_fewtok_kernel<NF, R, U, S, OUT, 3>), grd, blk, 0, s, e); break;
    }
}

template <int NF, int R, int U, int S>
static hipError_t launch(const GemmArgs& g, hipStream_t s) {
    Args a;
    a.vals = static_cast<const int8_t*>(g.values);
    a.meta = g.meta;
    a.X = static_cast<const int8_t*>(g.X);
    a.scale = g.scale;
    a.bias = g.bias;
    a.inv_scale = g.inv_scale;
    a.Y = g.Y;
    a.M = g.M; a.K = g.K; a.N = g.N; a.ldx = g.ldx; a.sxb = g.sx; a.ldy = g.ldy; a.syb = g.sy;
    a.y_vec = ((reinterpret_cast<uintptr_t>(g.Y) & 15) == 0) && g.ldy % 4 == 0 && (g.batch == 1 || g.sy % 4 == 0);
    const unsigned grid = (unsigned)(((g.M + 15) / 16 + R - 1) / R);
    // grid y covers at most 65535 batch entries per launch
    const int es = g.out_kind == OUT_BF16 ? 2 : (g.out_kind == OUT_I8 ? 1 : 4);
    const int epi = (g.bias ? 1 : 0) | (g.gelu ? 2 : 0);
    for (int64_t e0 = 0; e0 < g.batch; e0 += 65535) {
        const unsigned gb = (unsigned)(g.batch - e0 < 65535 ? g.batch - e0 : 65535);
        Args e = a;
        e.X = a.X + e0 * a.sxb;
        e.Y = static_cast<char*>(a.Y) + e0 * a.syb * es;
        const dim3 grd(grid, gb), blk(64 * S);
        switch (g.out_kind) {
        case OUT_I32: hipLaunchKernelGGL((gemm_i8_fewtok_kernel<NF, R, U, S, OUT_I32, 0>), grd, blk, 0, s, e); break;
        case OUT_F32: launch_epi<NF, R, U, S, OUT_F32>(epi, grd, blk, s, e); break;
        case OUT_BF16: launch_epi<NF, R, U, S, OUT_BF16>(epi, grd, blk, s, e); break;
        default: launch_epi<NF, R, U, S, OUT_I8>(epi, grd, blk, s, e); break;
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace fewtok_i8

bool gemm_i8_fewtok_ok(const GemmArgs& g) {
    // raw int32 accumulators without a scale, every epilogue with one; 16-byte aligned rows of X in every
    // batch entry; whole 128-column tiles; 32-bit byte offsets for X and for R = 4 row blocks' tiles
    const bool epi_ok = g.scale ? true : (g.out_kind == OUT_I32 && !g.bias && !g.gelu);
    const bool aligned = g.ldx % 16 == 0 && (reinterpret_cast<uintptr_t>(g.X) & 15) == 0 && (g.batch == 1 || g.sx % 16 == 0);
    return g.tm && epi_ok && aligned && g.N >= 1 && g.N <= 64 && g.K >= fewtok_i8::KT && g.K % fewtok_i8::KT == 0 &&
           (g.N - 1) * g.ldx + g.K + 128 < ((int64_t)1 << 31) && 4 * (g.K / fewtok_i8::KT) * 1024 < ((int64_t)1 << 31);
}

// Row blocks per workgroup (R), tiles per request round (U) and waves (S) by the number of 16-token
// fragments, measured on MI355X (HIP graph replays, weight copies rotated beyond the Infinity Cache) over
// R in {1, 2, 4, 8}, U in {1, 2, 4, 8}, S in {4, 8, 16}: U = 4, S = 8 up to two fragments and S = 4 beyond.
// R = 2 where it still gives over 256 workgroups (4096 x 4096 / 11008 x 4096 / 28672 x 8192 at N = 64:
// 12.8 / 21.5 / 69.6 us, against 12.1 / 27.7 / 69.6 with R = 1); R = 1 below that, and for one fragment
// up to 1024 row blocks, where the wider grid keeps more requests in flight (N = 1: 5.4 / 8.4 / 28.4 us,
// against 6.7 / 9.9 / 28.5 with R = 2).
hipError_t launch_gemm_i8_fewtok(const GemmArgs& g, hipStream_t s) {
    const int64_t nb = (g.M + 15) / 16;
    const int nf = (int)((g.N + 15) / 16);
    const bool r1 = nb <= 512 || (nf == 1 && nb <= 1024);
    switch (nf) {
    case 1: return r1 ? fewtok_i8::launch<1, 1, 4, 8>(g, s) : fewtok_i8::launch<1, 2, 4, 8>(g, s);
    case 2: return r1 ? fewtok_i8::launch<2, 1, 4, 8>(g, s) : fewtok_i8::launch<2, 2, 4, 8>(g, s);
    case 3: return r1 ? fewtok_i8::launch<3, 1, 4, 4>(g, s) : fewtok_i8::launch<3, 2, 4, 4>(g, s);
    default: return r1 ? fewtok_i8::launch<4, 1, 4, 4>(g, s) : fewtok_i8::launch<4, 2, 4, 4>(g, s);
    }
}

}  // namespace sp24
