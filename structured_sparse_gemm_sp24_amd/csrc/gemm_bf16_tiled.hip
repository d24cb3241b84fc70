// Tiled sparse x dense GEMM for large N, bf16 in, fp32 accumulate (NVIDIA blog on Ampere structured
// sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1 Step 3).
//
// Workgroup tile 256 (M) x 256 (N), 4 waves in a 2 x 2 grid, each wave 128 x 128 = 8 x 8
// v_smfmac_f32_16x16x64_bf16 fragments (256 fp32 accumulators per lane, one wave per SIMD).
// K advances 64 dense columns per stage; three stages are in flight through LDS (3 x 50 KB).
//
// Global -> LDS uses buffer loads with LDS destination (no VGPR staging); the buffer descriptors'
// record counts return zeros past the padded rows and past the end of X, so M/N tails need no
// branches in the main loop (columns past N only feed output columns that are never stored).
//   A (compressed values): the weight is stored as 1 KB tiles in the lane order of the smfmac A
//     operand (16 rows x 64 dense columns), so each tile is one contiguous 64-lane copy, and a
//     lane's ds_read_b128 of its operand is conflict-free.
//   metadata: 128 B tiles in lane order; a lane reads its 16-bit index with ds_read_u16.
//   B tile (X, 64 rows x 256 bf16 = 512 B per row): row-major with the 64-byte blocks of row k
//     stored at block ^ (k & 3), so the transposing reads below hit distinct banks while every
//     global read stays a run of 64 contiguous bytes.
// The B operand (lane = column, 16 k values in two halves of 8) comes from four ds_read_b64_tr_b16:
// in each 16-lane group, lane s points at row k0 + s/4, columns c0 + 4(s%4); the instruction hands
// lane i the four consecutive k of column c0 + i.
//
// Tiles are ordered XCD-first: workgroup p runs on XCD p % 8, so logical tiles are numbered such
// that each XCD gets a contiguous range, walked in groups of 8 tile-rows (A tiles and B tiles are
// re-read from that XCD's L2).
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace tiled_bf16 {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WM = 128, WN = 128;
constexpr int FM = WM / 16, FN = WN / 16;
constexpr int A_BYTES = BM * BK;          // BK/2 bf16 values per row = BK bytes
constexpr int META_BYTES = BM * BK / 8;   // 4 bits per group of 4
constexpr int B_BYTES = BK * BN * 2;
constexpr int B_ROW = BN * 2;             // 512 bytes
constexpr int STAGE_BYTES = A_BYTES + META_BYTES + B_BYTES;
constexpr int LOADS_PER_STAGE = 4 + 2 + 8;  // per wave: A, metadata, B
constexpr int GROUP_M = 8;
constexpr uint32_t RSRC_FLAGS = 0x00020000u;

// Raw buffer descriptor: base, stride 0, byte count (reads at or past it return 0), format word.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)n);
    r[3] = (int)RSRC_FLAGS;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// Buffer loads with LDS destination: lane i's bytes land at lds + i * width. Issued from inline asm
// so the compiler adds no waits of its own for them; the kernel orders them with explicit
// s_waitcnt vmcnt + s_barrier. They write no VGPRs.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform (it depends on the wave index only)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct Args {
    const uint16_t* vals;
    const uint8_t* meta;
    const uint16_t* X;
    void* Y;
    int64_t M, K, N, ldx, ldy;
    int tilesM, tilesN;
    int out_fp32;
};

// Issue this wave's share of the loads of stage `s` into `smem`. rA / rM cover the compressed
// tiles of this workgroup's 16 row blocks (tile (b, s) of block b at (b * tiles + s) * 1 KB of
// values and * 128 B of metadata); loads past the padded rows return zeros.
__device__ __forceinline__ void load_stage(char* smem, const Args& a, i32x4 rA, i32x4 rM, int64_t n0, int s,
                                           int wave, int lane) {
    const int64_t k0 = (int64_t)s * BK;
    const int tiles = (int)(a.K / BK);
    // A: one 1 KB tile per 16-row block, copied as is (it is already in lane order)
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int b = 4 * wave + j;
        dma16(lds_addr(smem + b * 1024), (uint32_t)((b * tiles + s) * 1024 + 16 * lane), rA);
    }
    // metadata: one 128 B tile per block; 4 blocks per wave, two per dword instruction
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int b = 4 * wave + 2 * h + (lane >> 5);
        dma4(lds_addr(smem + A_BYTES + (4 * wave + 2 * h) * 128), (uint32_t)((b * tiles + s) * 128 + 4 * (lane & 31)),
             rM);
    }
    // B: 64 rows x 512 B; this wave loads rows 16*wave .. +15, two rows per instruction. The 64-byte
    // blocks of row k are stored at block ^ (k & 3); lanes keep 16-byte runs in order inside a block.
    const i32x4 rB = make_rsrc(a.X + k0 * a.ldx + n0, (a.K * a.ldx - k0 * a.ldx - n0) * 2);
#pragma unroll
    for (int h = 0; h < 8; h++) {
        const int row = 16 * wave + 2 * h + (lane >> 5);
        const int pc = lane & 31;                                  // 16-byte slot in the LDS row
        const int lc = ((((pc >> 2) ^ (row & 3))) << 2) | (pc & 3);  // 16-byte chunk of the X row
        dma16(lds_addr(smem + A_BYTES + META_BYTES + (16 * wave + 2 * h) * B_ROW),
              (uint32_t)(row * a.ldx * 2 + 16 * lc), rB);
    }
}

// Lane-dependent LDS byte offsets used by compute_stage (computed once per kernel).
struct LaneOffsets {
    int a;        // A fragment of block wm0/16: block * 1024 + lane * 16
    int m;        // metadata of block wm0/16: A_BYTES + block * 128 + lane * 2
    int b[FN];    // B fragment j, first read (t = 0): row part + swizzled column part
};

__device__ __forceinline__ LaneOffsets lane_offsets(int wm0, int wn0, int lane) {
    const int r = lane & 15, q = lane >> 4;
    LaneOffsets o;
    o.a = (wm0 >> 4) * 1024 + lane * 16;
    o.m = A_BYTES + (wm0 >> 4) * 128 + lane * 2;
    // read t of group q covers rows 8q + 4(t&1) + 32(t>>1) + r/4; row & 3 = (r >> 2) & 3 fixes the
    // block swizzle for every t, so t only adds immediates
    const int row0 = 8 * q + (r >> 2);
    const int sw = row0 & 3;
#pragma unroll
    for (int j = 0; j < FN; j++) {
        const int col = wn0 + 16 * j + 4 * (r & 3);  // first of the 4 columns this lane points at
        o.b[j] = A_BYTES + META_BYTES + row0 * B_ROW + (((col >> 5) ^ sw) << 6) + 2 * (col & 31);
    }
    return o;
}

__device__ __forceinline__ void compute_stage(const char* smem, f32x4 (&acc)[FM][FN], const LaneOffsets& o) {
    bf16x8 a[FM];
    uint32_t idx[FM];
#pragma unroll
    for (int i = 0; i < FM; i++) {
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + o.a + i * 1024));
        idx[i] = *reinterpret_cast<const uint16_t*>(smem + o.m + i * 128);
    }
#pragma unroll
    for (int j = 0; j < FN; j++) {
        u32x8 b;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            // t = 0, 1: rows 8q + 4t + r/4; t = 2, 3: the same + 32
            const int imm = (t & 1) * 4 * B_ROW + (t >> 1) * 32 * B_ROW;
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(smem + o.b[j] + imm));
            b[2 * t] = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
            b[2 * t + 1] = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
        }
        const bf16x16 bb = __builtin_bit_cast(bf16x16, b);
#pragma unroll
        for (int i = 0; i < FM; i++)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a[i], bb, acc[i][j], (int)idx[i], 0, 0);
    }
}

template <int CUR, int STAGES>
__device__ __forceinline__ void step(char* cur, char* nxt, const Args& a, i32x4 rA,
                                     i32x4 rM, int64_t n0, int s, int S, f32x4 (&acc)[FM][FN],
                                     const LaneOffsets& o, int wave, int lane) {
    if (s + 2 < S) {
        load_stage(nxt, a, rA, rM, n0, s + 2, wave, lane);
        wait_vmcnt<2 * LOADS_PER_STAGE>();
    } else if (s + 1 < S) {
        wait_vmcnt<LOADS_PER_STAGE>();
    } else {
        wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    compute_stage(cur, acc, o);
    __builtin_amdgcn_s_barrier();
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_tiled_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) char s0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char s1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char s2[STAGE_BYTES];

    // XCD-first, then grouped tile order
    const int T = a.tilesM * a.tilesN;
    const int pid = blockIdx.x;
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = T >> 3, rem = T & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int gsize = GROUP_M * a.tilesN;
    const int g = logical / gsize;
    const int first_m = g * GROUP_M;
    const int gm = (a.tilesM - first_m) < GROUP_M ? (a.tilesM - first_m) : GROUP_M;
    const int in_g = logical - g * gsize;
    const int tm = first_m + in_g % gm, tn = in_g / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    // compressed tiles of this workgroup's first row block onward (rows are padded to 16)
    const int64_t tiles = a.K / BK, blocks_left = (a.M + 15) / 16 - m0 / 16;
    const i32x4 rA = make_rsrc(reinterpret_cast<const char*>(a.vals) + (m0 / 16) * tiles * 1024,
                               blocks_left * tiles * 1024);
    const i32x4 rM = make_rsrc(a.meta + (m0 / 16) * tiles * 128, blocks_left * tiles * 128);

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const LaneOffsets o = lane_offsets(wm0, wn0, lane);
    const int S = (int)(a.K / BK);
    load_stage(s0, a, rA, rM, n0, 0, wave, lane);
    if (S > 1) load_stage(s1, a, rA, rM, n0, 1, wave, lane);
    // main loop in groups of three stages (one per LDS buffer), then the 0-2 remaining stages;
    // keeping the loop body free of early exits keeps the accumulators in registers
    int s = 0;
    for (; s + 3 <= S; s += 3) {
        step<0, 3>(s0, s2, a, rA, rM, n0, s, S, acc, o, wave, lane);
        step<1, 3>(s1, s0, a, rA, rM, n0, s + 1, S, acc, o, wave, lane);
        step<2, 3>(s2, s1, a, rA, rM, n0, s + 2, S, acc, o, wave, lane);
    }
    if (s < S) step<0, 3>(s0, s2, a, rA, rM, n0, s, S, acc, o, wave, lane);
    if (s + 1 < S) step<1, 3>(s1, s0, a, rA, rM, n0, s + 1, S, acc, o, wave, lane);

    // epilogue: lane holds column n0 + wn0 + 16 j + r, rows m0 + wm0 + 16 i + 4 q + t
    const int r = lane & 15, q = lane >> 4;
    const int64_t mrow = m0 + wm0 + 4 * q, ncol = n0 + wn0 + r;
    const bool full = (m0 + BM <= a.M) && (n0 + BN <= a.N);
    if (a.out_fp32) {
        float* y = reinterpret_cast<float*>(a.Y) + mrow * a.ldy + ncol;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    if (full || (mrow + 16 * i + t < a.M && ncol + 16 * j < a.N))
                        y[(16 * i + t) * a.ldy + 16 * j] = acc[i][j][t];
    } else {
        uint16_t* y = reinterpret_cast<uint16_t*>(a.Y) + mrow * a.ldy + ncol;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    if (full || (mrow + 16 * i + t < a.M && ncol + 16 * j < a.N))
                        y[(16 * i + t) * a.ldy + 16 * j] = f32_to_bf16_rne(acc[i][j][t]);
    }
}

}  // namespace tiled_bf16

bool gemm_bf16_tiled_ok(int64_t M, int64_t K, int64_t N, int64_t ldx, const void* X) {
    return K % tiled_bf16::BK == 0 && ldx % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0 && N > 64 &&
           ldx < ((int64_t)1 << 24) && K < ((int64_t)1 << 24) && ((M + 255) / 256) * ((N + 255) / 256) < (1 << 30);
}

hipError_t launch_gemm_bf16_tiled(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                                  int64_t N, int64_t ldx, void* Y, bool out_fp32, int64_t ldy, hipStream_t s) {
    tiled_bf16::Args a;
    a.vals = values; a.meta = meta; a.X = X; a.Y = Y;
    a.M = M; a.K = K; a.N = N; a.ldx = ldx; a.ldy = ldy;
    a.tilesM = (int)((M + tiled_bf16::BM - 1) / tiled_bf16::BM);
    a.tilesN = (int)((N + tiled_bf16::BN - 1) / tiled_bf16::BN);
    a.out_fp32 = out_fp32 ? 1 : 0;
    const unsigned grid = (unsigned)(a.tilesM * a.tilesN);
    hipLaunchKernelGGL(tiled_bf16::gemm_bf16_tiled_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sp24
