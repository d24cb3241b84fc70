// Sparse x dense int8 GEMM for a few tokens in the Linear layout (token-major X, N <= 64), exact int32
// accumulation, the optional per-output-channel fp32 dequant and the fused FFN epilogue (bias, GELU, bf16
// or requantized int8 output) (oeforum post on sparse acceleration: int8 and 2:4 combine; NVIDIA blog on
// Ampere structured sparsity, Figure 1 and its quantization section; Orin NN design, Chapter 7, section
// 3.1 Step 4).
//
// With N this small the product streams the compressed int8 weight (0.625 bytes per dense weight) from
// HBM once, and X (N rows of K bytes) stays in L2. Two main loops share the reduction and the epilogue:
// up to 16 tokens an LDS ring (gemm_i8_fewtok_ring, described there) keeps several K tiles in flight per
// wave; otherwise a register-pipelined loop. In the latter a workgroup owns R consecutive 16-row blocks and
// all N tokens (NF fragments of 16); its S waves split the K tiles (128 dense columns each) into contiguous
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

// The waves' partial sums through LDS (red: (S - 1) * R * NF * 64 i32x4, workgroup-shared), then wave 0's
// value pipeline and stores.
template <int NF, int R, int S, int OUT, int EPI>
__device__ __forceinline__ void finish(i32x4 (&acc)[R][NF], const Args& a, i32x4* red, int64_t b0, int wave,
                                       int lane) {
    const int r = lane & 15, q = lane >> 4;
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


// LDS-destination buffer loads (lane i's bytes land at lds + i * width), from inline asm so the compiler adds
// no waits of its own; the whole byte offset is the VGPR operand, which the range check covers.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
                 : "memory");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Raw descriptor as four words (for the asm loads): base, stride 0, byte count, format word.
__device__ __forceinline__ i32x4 rsrc4(const void* base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes);
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)n);
    r[3] = 0x00020000;
    return r;
}
// 16-byte unit swizzle of token row n of an X tile in LDS: the 16 lanes of one read group (tokens 0..15, one
// unit each) fall in distinct 16-byte bank slots per row parity.
__device__ __forceinline__ int x_swz(int n) { return ((n >> 1) & 7) ^ ((n & 1) << 2); }

// One fragment of tokens (N <= 16) through a per-wave LDS ring: a workgroup owns one 16-row block and its S
// waves split the K tiles into contiguous ranges; each wave keeps D units in LDS, a unit being one K tile's
// compressed value tile (1 KB), index tile (256 B) and X tile (XR token rows of 128 B, 16-byte units of row n at
// unit ^ x_swz(n)), all landed by LDS-destination loads with a fixed count per unit. The wave issues unit
// i + D - 1 into the slot unit i - 1 has left, waits (vmcnt) until unit i has landed and multiplies it, so D - 1
// units stay in flight and no wave waits for another until the final reduction. Units past the wave's range
// read zeros without memory traffic (offset bit 31); tokens past N read zeros from the descriptor's range.
template <int S, int D, int XR, int R, int OUT, int EPI>
__global__ __launch_bounds__(64 * S) void gemm_i8_fewtok_ring(Args a) {
    static_assert(XR == 2 || XR == 8 || XR == 16, "X tile rows");
    constexpr int NXI = XR == 16 ? 2 : 1;  // X loads per unit (XR = 2: one dword load for both rows)
    // a unit: the K tile's R value tiles, their R index tiles, then the X tile all R blocks share
    constexpr int MOFF = 1024 * R, XOFF = 1280 * R, UNIT = XOFF + 128 * XR, RING = D * UNIT, LPU = 2 * R + NXI;
    constexpr int RED = (S - 1) * R * 64 * 16;
    static_assert((D - 1) * LPU < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) char smem[S * RING > RED ? S * RING : RED];
    typedef __attribute__((address_space(3))) char lds_char;
    typedef const __attribute__((address_space(3))) i32x4 lds_i32x4;
    const uint32_t l0 = (uint32_t)(size_t)(lds_char*)smem;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t b0 = (int64_t)blockIdx.x * R, nblk = (a.M + 15) / 16;
    const int T = (int)(a.K / KT);
    const int per = (T + S - 1) / S, t0 = wave * per, t1 = t0 + per < T ? t0 + per : T;
    const int n = t1 > t0 ? t1 - t0 : 0;
    // the workgroup's blocks (fewer in the last one: blocks past the weight read zeros)
    const int64_t nb = nblk - b0 < R ? nblk - b0 : R;
    const i32x4 rA = rsrc4(a.vals + b0 * T * 1024, nb * T * 1024);
    const i32x4 rM = rsrc4(a.meta + b0 * T * 256, nb * T * 256);
    const int8_t* X = a.X + (int64_t)blockIdx.y * a.sxb;
    const i32x4 rX = rsrc4(X, (a.N - 1) * a.ldx + a.K);
    // per-lane load offsets: value tile 16 * lane, index tile 4 * lane; X: 16-byte loads put lane i in row
    // 8h + i / 8, slot i % 8, which holds unit (i % 8) ^ x_swz(row); the dword load (XR = 2) puts lane i in row
    // i / 32, dword i % 32 of the row, i.e. dword i % 4 of slot (i % 32) / 4
    const uint32_t oA = 16u * (uint32_t)lane, oM = 4u * (uint32_t)lane;
    uint32_t oX[NXI];
    if constexpr (XR == 2) {
        const int row = lane >> 5, slot = (lane & 31) >> 2;
        oX[0] = (uint32_t)(row * a.ldx + 16 * (slot ^ x_swz(row)) + 4 * (lane & 3));
    } else {
#pragma unroll
        for (int h = 0; h < NXI; h++) {
            const int row = 8 * h + (lane >> 3);
            oX[h] = (uint32_t)(row * a.ldx + 16 * ((lane & 7) ^ x_swz(row)));
        }
    }
    const uint32_t ring = l0 + (uint32_t)(wave * RING);
    auto issue = [&](int i) {
        const uint32_t t = (uint32_t)(t0 + i), past = i < n ? 0u : OOR;
        const uint32_t slot = ring + (uint32_t)((i % D) * UNIT);
#pragma unroll
        for (int j = 0; j < R; j++) {
            const uint32_t tj = (uint32_t)(j * T) + t;
            dma16(slot + 1024 * j, (oA + tj * 1024u) | past, rA);
            dma4(slot + MOFF + 256 * j, (oM + tj * 256u) | past, rM);
        }
        if constexpr (XR == 2) {
            dma4(slot + XOFF, (oX[0] + t * (uint32_t)KT) | past, rX);
        } else {
#pragma unroll
            for (int h = 0; h < NXI; h++) dma16(slot + XOFF + 1024 * h, (oX[h] + t * (uint32_t)KT) | past, rX);
        }
    };
    // lane (r, q) reads its value and index operands, and token row r's units q and q + 4 (rows past the tile's
    // XR feed only tokens >= XR > N - 1, never stored: any row of the tile will do)
    const int xr = r & (XR - 1);
    const int xo0 = XOFF + xr * 128 + 16 * (q ^ x_swz(xr)), xo1 = XOFF + xr * 128 + 16 * ((q ^ x_swz(xr)) ^ 4);
    i32x4 acc[R][1];
#pragma unroll
    for (int j = 0; j < R; j++) acc[j][0] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < D - 1; i++) issue(i);
    for (int i = 0; i < n; i++) {
        issue(i + D - 1);              // into the slot unit i - 1 has left (its reads completed before its smfmac)
        wait_vmcnt<(D - 1) * LPU>();  // unit i has landed
        asm volatile("" ::: "memory");
        const lds_char* p = (const lds_char*)(size_t)(ring + (uint32_t)((i % D) * UNIT));
        const i32x4 lo = *reinterpret_cast<lds_i32x4*>(p + xo0), hi = *reinterpret_cast<lds_i32x4*>(p + xo1);
        const i32x8 bx = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int j = 0; j < R; j++) {
            const i32x4 av = *reinterpret_cast<lds_i32x4*>(p + 1024 * j + 16 * lane);
            const int iv = *reinterpret_cast<const __attribute__((address_space(3))) int*>(p + MOFF + 256 * j + 4 * lane);
            acc[j][0] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bx, acc[j][0], iv, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this unit's reads are done before its slot is refilled
    }
    wait_vmcnt<0>();  // every load (the zero-filling ones included) has landed before LDS is reused
    __syncthreads();  // every wave is done with its ring
    finish<1, R, S, OUT, EPI>(acc, a, reinterpret_cast<i32x4*>(smem), b0, wave, lane);
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

    finish<NF, R, S, OUT, EPI>(acc, a, red, b0, wave, lane);
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

template <int S, int D, int XR, int R, int OUT>
static void launch_ring_epi(int epi, dim3 grd, dim3 blk, hipStream_t s, const Args& e) {
    switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_i8_fewtok_ring<S, D, XR, R, OUT, 0>), grd, blk, 0, s, e); break;
    case 1: hipLaunchKernelGGL((gemm_i8_fewtok_ring<S, D, XR, R, OUT, 1>), grd, blk, 0, s, e); break;
    case 2: hipLaunchKernelGGL((gemm_i8_fewtok_ring<S, D, XR, R, OUT, 2>), grd, blk, 0, s, e); break;
    default: hipLaunchKernelGGL((gemm_i8_fewtok_ring<S, D, XR, R, OUT, 3>), grd, blk, 0, s, e); break;
    }
}

// The LDS-ring kernel (N <= XR <= 16): R 16-row blocks per workgroup.
template <int S, int D, int XR, int R = 1>
static hipError_t launch_ring(const GemmArgs& g, hipStream_t s) {
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
    const int es = g.out_kind == OUT_BF16 ? 2 : (g.out_kind == OUT_I8 ? 1 : 4);
    const int epi = (g.bias ? 1 : 0) | (g.gelu ? 2 : 0);
    for (int64_t e0 = 0; e0 < g.batch; e0 += 65535) {
        const unsigned gb = (unsigned)(g.batch - e0 < 65535 ? g.batch - e0 : 65535);
        Args e = a;
        e.X = a.X + e0 * a.sxb;
        e.Y = static_cast<char*>(a.Y) + e0 * a.syb * es;
        const dim3 grd(grid, gb), blk(64 * S);
        switch (g.out_kind) {
        case OUT_I32: hipLaunchKernelGGL((gemm_i8_fewtok_ring<S, D, XR, R, OUT_I32, 0>), grd, blk, 0, s, e); break;
        case OUT_F32: launch_ring_epi<S, D, XR, R, OUT_F32>(epi, grd, blk, s, e); break;
        case OUT_BF16: launch_ring_epi<S, D, XR, R, OUT_BF16>(epi, grd, blk, s, e); break;
        default: launch_ring_epi<S, D, XR, R, OUT_I8>(epi, grd, blk, s, e); break;
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace fewtok_i8

bool gemm_i8_fewtok_ok(const GemmArgs& g) {
    // raw int32 accumulators without a scale, every epilogue with one; 16-byte aligned rows of X in every
    // batch entry; whole 128-column tiles; 32-bit byte offsets for X and for R = 8 row blocks' tiles
    const bool epi_ok = g.scale ? true : (g.out_kind == OUT_I32 && !g.bias && !g.gelu);
    const bool aligned = g.ldx % 16 == 0 && (reinterpret_cast<uintptr_t>(g.X) & 15) == 0 && (g.batch == 1 || g.sx % 16 == 0);
    return g.tm && epi_ok && aligned && g.N >= 1 && g.N <= 64 && g.K >= fewtok_i8::KT && g.K % fewtok_i8::KT == 0 &&
           (g.N - 1) * g.ldx + g.K + 128 < ((int64_t)1 << 31) && 8 * (g.K / fewtok_i8::KT) * 1024 < ((int64_t)1 << 31);
}

// The register loop with R = r row blocks per workgroup for r in [RMIN, RMAX] (RMAX otherwise).
template <int NF, int U, int S, int RMIN, int RMAX>
static hipError_t launch_r(const GemmArgs& g, hipStream_t s, int64_t r) {
    if constexpr (RMIN <= 3 && RMAX >= 3) if (r == 3) return fewtok_i8::launch<NF, 3, U, S>(g, s);
    if constexpr (RMIN <= 4 && RMAX > 4) if (r == 4) return fewtok_i8::launch<NF, 4, U, S>(g, s);
    if constexpr (RMIN <= 5 && RMAX > 5) if (r == 5) return fewtok_i8::launch<NF, 5, U, S>(g, s);
    if constexpr (RMIN <= 6 && RMAX > 6) if (r == 6) return fewtok_i8::launch<NF, 6, U, S>(g, s);
    if constexpr (RMIN <= 7 && RMAX > 7) if (r == 7) return fewtok_i8::launch<NF, 7, U, S>(g, s);
    return fewtok_i8::launch<NF, RMAX, U, S>(g, s);
}

// Register loop: row blocks per workgroup (R), tiles per request round (U) and waves (S) by the number of 16-token
// fragments and of row blocks, measured on MI355X with weight copies rotated beyond the Infinity Cache over
// R in {1, 2, 4, 8}, U in {1, 2, 4}, S in {4, 8}. More row blocks per workgroup share each X fragment; the best
// grid is about one round of workgroups (28672 x 8192 at N = 64 / 32: 69.4 / 43.8 -> 47.8 / 35.7 us with R = 4 /
// 8; 11008 x 4096 at N = 64 / 32: 21.2 / 15.0 -> 18.2 / 12.4 us with R = 4; 6144 x 4096 at N = 64 19.4 -> 12.9
// us with R = 2), and two tiles per round beat four at one fragment below 1024 blocks (11008 x 4096 at N = 8:
// 8.9 -> 8.2 us; 4096 x 4096 at N = 8 5.0 -> 4.8 us).
hipError_t launch_gemm_i8_fewtok(const GemmArgs& g, hipStream_t s) {
    const int64_t nb = (g.M + 15) / 16;
    const int nf = (int)((g.N + 15) / 16);
    // the LDS ring: one or two tokens on weights of 1024 row blocks and more, 9 to 16 tokens below that
    // (24 rotated copies, beyond the Infinity Cache: 16400 x 4096 at N = 1 11.9 -> 11.0 us; 11008 x 4096 at
    // N = 16 10.6 -> 9.9 us; 4096 x 4096 at N = 16 5.5 -> 4.9 us; 6144 x 4096 at N = 12 7.4 -> 7.2 us). The
    // register loop stays for 3 to 8 tokens (11008 x 4096 at N = 3 / 4 / 6 / 8: 8.0 / 7.9 / 8.6 / 9.2 against
    // 8.5 / 8.2 / 8.7 / 8.9 us), for N <= 2 below 1024 blocks and for N > 8 from 1024 (28672 x 8192 at N = 16:
    // 32.7 against 35.4 us). Workgroups of 4 waves (three per CU) from 512 blocks, of 8 (two per CU) below.
    if (g.N <= 2 && nb >= 1024) return fewtok_i8::launch_ring<4, 8, 2>(g, s);  // 48 KB
    if (g.N > 8 && g.N <= 16 && nb < 1024) {
        // three or four row blocks per unit, sharing its X tile, where that makes a round of at least 7/8 of
        // the CUs (bit-identical; 11008 x 4096 at N = 16 / 12 9.84 / 9.74 -> 9.28 / 9.22 us with three, 16000 x
        // 4096 and 14336 x 4096 at N = 16 12.97 / 12.0 -> 12.32 / 11.5 with four; 12290 x 4096, 193 workgroups
        // of four, 9.96 -> 10.38, so not there): one 94 / 115 KB workgroup per CU
        const int64_t cus = device_cus();
        if (nb > 2 * cus && 8 * ((nb + 2) / 3) >= 7 * cus && nb <= 3 * cus) return fewtok_i8::launch_ring<4, 4, 16, 3>(g, s);
        if (8 * ((nb + 3) / 4) >= 7 * cus && nb <= 4 * cus) return fewtok_i8::launch_ring<4, 4, 16, 4>(g, s);
        return nb >= 512 ? fewtok_i8::launch_ring<4, 4, 16>(g, s) : fewtok_i8::launch_ring<8, 3, 16>(g, s);  // 52 / 78 KB
    }
    using namespace fewtok_i8;
    // register loop: R row blocks per workgroup. From 512 to 1024 row blocks (and 17 to 32 tokens beyond),
    // R = ceil(blocks / CUs) loads every CU alike in one round (bit-identical; 11008 x 4096 at N = 24 / 40 /
    // 64 11.9 / 15.4 / 18.2 -> 11.5 / 14.1 / 16.9 us with R = 3 instead of 4, 8200 x 4096 at N = 64 17.7 ->
    // 16.4, 16384 x 4096 at N = 12 17.2 -> 15.3 with R = 4 instead of 8, 28672 x 8192 at N = 32 36.3 -> 35.2
    // with R = 7). On 28672 x 8192 at one or three to four fragments the earlier grids stream faster (N = 16:
    // 32.8 against 39.9 us with R = 7; N = 64: 49.0 against 58.3) and stay.
    const int64_t cus = device_cus(), r = (nb + cus - 1) / cus;
    if (nf == 1) {
        if (nb >= 1024) {
            if (g.N <= 8) return launch<1, 2, 4, 8>(g, s);
            return r == 4 ? launch<1, 4, 4, 8>(g, s) : launch<1, 8, 4, 8>(g, s);
        }
        return nb >= 512 ? launch<1, 1, 2, 4>(g, s) : launch<1, 1, 2, 8>(g, s);
    }
    if (nf == 2) {
        if (nb > 1024) return r <= 8 ? launch_r<2, 2, 8, 5, 8>(g, s, r) : launch<2, 8, 2, 8>(g, s);
        if (nb > 512) return launch_r<2, 2, 4, 3, 4>(g, s, r);
        if (nb > 256) return launch<2, 2, 2, 8>(g, s);
        return launch<2, 1, 2, 4>(g, s);
    }
    if (nf == 3) {
        if (nb > 1024) return launch<3, 4, 4, 4>(g, s);
        if (nb > 512) return launch_r<3, 2, 8, 3, 4>(g, s, r);
        if (nb > 256) return launch<3, 2, 4, 4>(g, s);
        return launch<3, 1, 2, 4>(g, s);
    }
    if (nb > 1024) return launch<4, 4, 4, 4>(g, s);
    if (nb > 512) return launch_r<4, 2, 8, 3, 4>(g, s, r);
    if (nb > 256) return launch<4, 2, 4, 4>(g, s);
    return launch<4, 1, 2, 4>(g, s);
}

}  // namespace sp24
