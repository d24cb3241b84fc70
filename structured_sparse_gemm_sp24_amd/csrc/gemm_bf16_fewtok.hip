// Sparse x dense GEMM for a few tokens in the Linear layout (token-major X, N <= 16), bf16 in, fp32
// accumulate (NVIDIA blog on Ampere structured sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1
// Step 3).
//
// At such N the product streams the compressed weight (1.125 bytes per dense weight) from HBM once,
// and the time is set by how many of those bytes are in flight: HBM latency under load is a couple of
// microseconds, so a compute unit needs tens of KB outstanding. Here they wait in LDS, not in
// registers:
//  - a workgroup owns one 16-row block of the weight and all N tokens; its S waves split the block's
//    K tiles (64 dense columns each) into S contiguous ranges;
//  - each wave keeps a private ring of D units in LDS. A unit is one K tile: the 1 KB compressed value
//    tile (already in smfmac lane order), its 128-byte index tile, and the X tile (XR = 2, 8 or 16 token
//    rows x 128 bytes, 16-byte units of row n at unit ^ f(n) as in the tiled kernel's token-major B
//    tile), each fetched with LDS-destination buffer loads, so no VGPRs hold data in flight;
//  - the wave issues unit i + D - 1 into the slot that unit i - 1 has just left, waits (vmcnt) until
//    unit i has landed, and multiplies it: D - 1 units stay in flight, every unit issues the same
//    number of loads (units past the range are pushed out of the descriptor's range: zeros, no memory
//    traffic), and no wave waits for another until the end;
//  - token rows past N come back as zeros from the buffer range check (they only feed output columns
//    that are never stored); a partial last K tile is multiplied outside the ring with its X elements
//    read one by one, so nothing at k >= K (the next token's row, or row padding) is ever used;
//  - at the end the S partial 16 x 16 accumulators are summed through LDS in wave order
//    (deterministic), rounded if the output is bf16, and stored into Y (N x M) with bounds checks.
// A batch of products sharing the weight is grid dimension y.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace fewtok {

struct Args {
    const uint8_t* vals;
    const uint8_t* meta;
    int64_t M, K, N;
    const uint16_t* X;
    int64_t ldx, sxb;
    void* Y;
    int64_t ldy, syb;
    int out_fp32;
};

constexpr uint32_t RSRC_FLAGS = 0x00020000u;

// Raw buffer descriptor: base, stride 0, byte count rounded up to whole dwords, format word.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > 0xFFFFFFFCll ? 0xFFFFFFFCll : (bytes + 3) & ~(int64_t)3);
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)n);
    r[3] = (int)RSRC_FLAGS;
    return r;
}

// Buffer loads with LDS destination (lane i's bytes land at lds + i * width), from inline asm so the
// compiler adds no waits of its own; they write no VGPRs. The whole byte offset is in the VGPR operand,
// which the range check covers.
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

__device__ __forceinline__ int tm_swz(int n) { return ((n >> 1) & 7) ^ ((n & 1) << 2); }

typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int S, int D, int XR>
__global__ __launch_bounds__(64 * S) void gemm_bf16_fewtok(Args g) {
    static_assert(XR == 2 || XR == 8 || XR == 16, "X tile rows");
    constexpr int NXI = XR == 16 ? 2 : 1;           // X loads per unit (one dword load for 2 rows)
    constexpr int UNIT = 1024 + 256 + 128 * XR;     // value tile, index tile (128 B used), X tile
    constexpr int RING = D * UNIT;                  // per wave
    constexpr int LPU = 2 + NXI;                    // loads per unit
    constexpr int RED = S * 256 * 4;
    static_assert((D - 1) * LPU < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) char smem[S * RING > RED ? S * RING : RED];
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t M = g.M, K = g.K, N = g.N, ldx = g.ldx;
    const int64_t b = blockIdx.x;
    const uint16_t* const X = g.X + (int64_t)blockIdx.y * g.sxb;
    const int64_t T = (K + 63) / 64, Tf = K / 64;  // tiles per row block; full ones
    const int64_t t0 = T * wave / S, t1 = T * (wave + 1) / S;
    const int64_t tf = t1 < Tf ? t1 : Tf;         // the ring takes the full tiles [t0, tf)
    const int n = (int)(tf > t0 ? tf - t0 : 0);

    const i32x4 rA = make_rsrc(g.vals + b * T * 1024, T * 1024);
    const i32x4 rM = make_rsrc(g.meta + b * T * 128, T * 128);
    const i32x4 rX = make_rsrc(X, ((N - 1) * ldx + K) * 2);
    // per-lane load offsets: value tile 16 * lane; index tile 4 * lane for lanes < 32 (the other half
    // of the dword load is pushed out of range); X: 16-byte loads put lane i in row 8h + i / 8, unit
    // slot i % 8, which holds unit (i % 8) ^ f(row); the dword load (XR = 2) puts lane i in row i / 32,
    // dword i % 32 of the row, i.e. dword i % 4 of unit slot (i % 32) / 4
    const uint32_t oA = 16u * (uint32_t)lane;
    const uint32_t oM = lane < 32 ? 4u * (uint32_t)lane : 0x80000000u;
    uint32_t oX[NXI];
    if constexpr (XR == 2) {
        const int row = lane >> 5, slot = (lane & 31) >> 2;
        oX[0] = (uint32_t)(row * ldx * 2 + 16 * (slot ^ tm_swz(row)) + 4 * (lane & 3));
    } else {
#pragma unroll
        for (int h = 0; h < NXI; h++) {
            const int row = 8 * h + (lane >> 3);
            oX[h] = (uint32_t)(row * ldx * 2 + 16 * ((lane & 7) ^ tm_swz(row)));
        }
    }
    const uint32_t ring = l0 + (uint32_t)(wave * RING);

    // unit i of this wave (tile t0 + i) into slot i % D; past the wave's full tiles the offsets get
    // bit 31 (beyond every record count): zeros, no memory traffic
    auto issue = [&](int i) {
        const uint32_t t = (uint32_t)(t0 + i), past = i < n ? 0u : 0x80000000u;
        const uint32_t slot = ring + (uint32_t)((i % D) * UNIT);
        dma16(slot, (oA + t * 1024u) | past, rA);
        dma4(slot + 1024, (oM + t * 128u) | past, rM);
        if constexpr (XR == 2) {
            dma4(slot + 1280, (oX[0] + t * 128u) | past, rX);
        } else {
#pragma unroll
            for (int h = 0; h < NXI; h++) dma16(slot + 1280 + 1024 * h, (oX[h] + t * 128u) | past, rX);
        }
    };

    // lane (r, q) reads: value operand at 16 * lane, index at 2 * lane, X row r (rows past the tile's
    // XR feed only output columns >= XR > N - 1, never stored: any row of the tile will do)
    const int xr = r & (XR - 1);
    const int xo0 = 1280 + xr * 128 + 16 * (q ^ tm_swz(xr)), xo1 = 1280 + xr * 128 + 16 * ((q ^ tm_swz(xr)) ^ 4);

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D - 1; i++) issue(i);
    for (int i = 0; i < n; i++) {
        issue(i + D - 1);  // into the slot unit i - 1 has left (its reads completed before its smfmac)
        wait_vmcnt<(D - 1) * LPU>();  // unit i has landed
        asm volatile("" ::: "memory");  // and the reads of it stay below the wait
        const lds_char* p = (const lds_char*)(size_t)(ring + (uint32_t)((i % D) * UNIT));
        const u32x4 av = *reinterpret_cast<lds_u32x4*>(p + 16 * lane);
        const uint32_t idx = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(p + 1024 + 2 * lane);
        const u32x4 lo = *reinterpret_cast<lds_u32x4*>(p + xo0);
        const u32x4 hi = *reinterpret_cast<lds_u32x4*>(p + xo1);
        const bf16x16 bx = __builtin_bit_cast(bf16x16, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, av), bx, acc, (int)idx, 0, 0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this unit's reads are done before its slot is refilled
    }
    wait_vmcnt<0>();  // every load (including the zero-filling ones) has landed before LDS is reused

    // the partial last K tile (K % 64 != 0): operands read directly, X elements at k >= K as zero
    if (t1 > tf && Tf < T) {
        const int64_t t = Tf;
        const u32x4 av = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g.vals + (b * T + t) * 1024) + lane);
        const uint32_t idx = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(g.meta + (b * T + t) * 128) + lane);
        u32x8 bw = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < N) {
            const uint16_t* xrow = X + (int64_t)r * ldx;
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const int64_t k = 64 * t + 8 * q + (e & 7) + 32 * (e >> 3);
                const uint32_t v0 = k < K ? xrow[k] : 0u;
                const uint32_t v1 = k + 1 < K ? xrow[k + 1] : 0u;
                bw[e >> 1] = v0 | (v1 << 16);
            }
        }
        acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x16, bw),
                                                        acc, (int)idx, 0, 0);
    }

    // sum the S partial tiles in wave order: lane (r, q) holds column r, rows 4q .. 4q+3 of the block
    __syncthreads();  // every wave is done with its ring
    float* const red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 4; i++) red[wave * 256 + (4 * q + i) * 16 + r] = acc[i];
    __syncthreads();
    char* const Y = static_cast<char*>(g.Y) + (int64_t)blockIdx.y * g.syb * (g.out_fp32 ? 4 : 2);
    for (int e = threadIdx.x; e < 256; e += 64 * S) {
        // consecutive threads take consecutive rows m of one token row of Y (N x M)
        const int row = e % 16, col = e / 16;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < S; w++) s += red[w * 256 + row * 16 + col];
        const int64_t m = b * 16 + row;
        if (m < M && col < N) {
            const int64_t o = (int64_t)col * g.ldy + m;
            if (g.out_fp32)
                reinterpret_cast<float*>(Y)[o] = s;
            else
                reinterpret_cast<uint16_t*>(Y)[o] = f32_to_bf16_rne(s);
        }
    }
}

template <int S, int D, int XR>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
    Args a;
    a.vals = static_cast<const uint8_t*>(g.values);
    a.meta = g.meta;
    a.M = g.M; a.K = g.K; a.N = g.N;
    a.X = static_cast<const uint16_t*>(g.X);
    a.ldx = g.ldx; a.sxb = g.sx;
    a.Y = g.Y;
    a.ldy = g.ldy; a.syb = g.sy;
    a.out_fp32 = g.out_fp32;
    const unsigned grid = (unsigned)((g.M + 15) / 16);
    for (int64_t b0 = 0; b0 < g.batch; b0 += 65535) {
        const unsigned gb = (unsigned)(g.batch - b0 < 65535 ? g.batch - b0 : 65535);
        Args e = a;
        e.X = a.X + b0 * a.sxb;
        e.Y = static_cast<char*>(a.Y) + b0 * a.syb * (g.out_fp32 ? 4 : 2);
        hipLaunchKernelGGL((gemm_bf16_fewtok<S, D, XR>), dim3(grid, gb), dim3(64 * S), 0, s, e);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace fewtok

// Where this kernel is used: measured against the register-pipelined few-token kernel on MI355X (HIP
// graph replays, weight copies rotated beyond the Infinity Cache): for N <= 2 (28672 x 8192 at N = 1: 44.9
// against 48.7 us), for 3 to 8 tokens up to 256 and from 513 to 1023 row blocks (11008 x 4096 at N = 4 / 8:
// 11.4 / 12.2 against 11.9 / 12.0 us, 16000 x 4096 at N = 8 16.0 against 17.2; in between the register
// kernel's two-block workgroups fit one round and win: 5000 x 4096 at N = 8 8.6 -> 7.6 us, 7000 x 4096 at
// N = 4 8.5 -> 7.8, 6000 x 4096 at N = 6 8.8 -> 8.1, 4400 x 4096 at N = 3 7.6 -> 6.8), and for
// 9 to 16 tokens up to 256 row blocks, one workgroup per CU (4096 x 4096 at N = 9 / 12 / 16: 7.0 / 6.9 / 7.1
// against 7.6 / 7.2 / 7.9 us). With 16-row X tiles a unit carries twice the X bytes of its weight bytes, and
// past 256 blocks the register kernel, whose workgroups share each X fragment among several row blocks and
// fit one round, is faster (cold: 5000 x 4096 at N = 16 10.6 -> 9.0 us, 6000 x 4096 at N = 12 10.1 -> 8.5,
// 4400 x 4096 at N = 16 10.4 -> 8.8, 5600 x 2048 at N = 10 6.5 -> 5.8; 11008 x 4096 at N = 16 13.9 against
// 14.7).
bool gemm_bf16_fewtok_ok(const GemmArgs& g) {
    // token-major, rows of X 16-byte aligned in every batch entry; 32-bit load offsets below bit 31
    // (which marks the loads past a wave's range): 16 X rows plus K, the value tiles of one row block
    // (16 K bytes)
    const bool aligned = g.ldx % 8 == 0 && (reinterpret_cast<uintptr_t>(g.X) & 15) == 0 && (g.batch == 1 || g.sx % 8 == 0);
    const int64_t nb = (g.M + 15) / 16;
    const bool pays = g.N <= 2 || (g.N <= 8 && nb < 1024 && (nb <= 256 || nb > 512)) || (g.N <= 16 && nb <= 256);
    return g.tm && g.N >= 1 && pays && aligned && (16 * g.ldx + g.K) * 2 < ((int64_t)1 << 31) &&
           g.K < ((int64_t)1 << 26) && nb < ((int64_t)1 << 31);
}

// Waves per workgroup (S) and ring depth (D) by the number of 16-row blocks: enough workgroups that
// all of them are resident at once, and as many LDS slots in flight per compute unit as that allows. Above
// 256 blocks the 4-wave workgroups (three per CU) keep every workgroup in one round; the 8-wave ones (one
// per CU) would run a second round (cold caches: 6144 x 4096 at N = 1 / 4 / 8 9.1 / 9.9 / 10.6 -> 7.9 / 8.2 /
// 8.9 us; 8000 x 4096 at N = 8 11.6 -> 9.3 us).
hipError_t launch_gemm_bf16_fewtok(const GemmArgs& g, hipStream_t s) {
    const int64_t nb = (g.M + 15) / 16;
    if (g.N <= 2) {
        if (nb > 256) return fewtok::launch<4, 8, 2>(g, s);    // 48 KB per workgroup, three per CU
        if (nb >= 192) return fewtok::launch<8, 8, 2>(g, s);   // 96 KB
        return fewtok::launch<16, 6, 2>(g, s);                 // 144 KB
    }
    if (g.N > 8) {  // 16 token rows per unit, at most 256 row blocks
        if (nb >= 192) return fewtok::launch<8, 3, 16>(g, s);  // 78 KB
        return fewtok::launch<16, 2, 16>(g, s);                // 104 KB
    }
    if (nb > 256) return fewtok::launch<4, 5, 8>(g, s);        // 46 KB
    if (nb >= 192) return fewtok::launch<8, 5, 8>(g, s);       // 92 KB
    return fewtok::launch<16, 4, 8>(g, s);                     // 147 KB
}

}  // namespace sp24
