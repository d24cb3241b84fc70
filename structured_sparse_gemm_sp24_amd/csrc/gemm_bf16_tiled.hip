// Tiled sparse x dense GEMM for large N, bf16 in, fp32 accumulate (NVIDIA blog on Ampere structured
// sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1 Step 3).
//
// Workgroup tile 256 (M) x 256 (N), 4 waves in a 2 x 2 grid, each wave 128 x 128 = 8 x 8
// v_smfmac_f32_16x16x64_bf16 fragments (256 fp32 accumulators per lane, one wave per SIMD).
// K advances 64 dense columns per stage; three stages are in flight through LDS (3 x 50 KB).
//
// Global -> LDS uses buffer loads with LDS destination (no VGPR staging). The whole byte offset of
// each load is in its VGPR operand, which the buffer range check covers (the SGPR offset is not
// checked), so reads past this workgroup's row blocks and past the end of X return zeros without
// touching memory: M/N tails need no branches in the main loop (columns past N only feed output
// columns that are never stored), and the loads the pipeline issues past the last stage are pushed
// out of range on purpose.
//   A (compressed values): the weight is stored as 1 KB tiles in the lane order of the smfmac A
//     operand (16 rows x 64 dense columns), so each tile is one contiguous 64-lane copy, and a
//     lane's ds_read_b128 of its operand is conflict-free.
//   metadata: 128 B tiles in lane order; a lane reads its 16-bit index with ds_read_u16.
//   B tile (X, 64 rows x 256 bf16 = 512 B per row): row-major with the 32-byte units of row k
//     stored at unit ^ v(k), v(k) = 2 (k & 3) + ((k >> 3) & 1). One transposing read (below) takes
//     16 rows x 32 bytes, rows 8q + {0..3} for q = 0..3; v puts them in 8 distinct 32-byte bank
//     groups (two rows each, the minimum for 512 bytes). In global memory every 4 consecutive lanes
//     of a load still read one aligned 64-byte run (v only swaps its two halves or moves it whole).
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

// Raw buffer descriptor: base, stride 0, byte count rounded up to whole dwords, format word. The range
// check returns a dword only when all of it is below the record count; the rounding keeps the last
// partial dword of the real data (that dword lies in the same page as the data it ends).
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


// Buffer loads with LDS destination: lane i's bytes land at lds + i * width. Issued from inline asm
// so the compiler adds no waits of its own for them; the kernel orders them with explicit
// s_waitcnt vmcnt + s_barrier. They write no VGPRs. `lds` is wave-uniform (an SGPR); `voff` is the
// lane's whole byte offset from the descriptor base (range-checked against its record count).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4 rsrc) {
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
    int y_vec;  // Y base and row pitch allow 16-byte stores
};

// Per-lane parts of the load offsets (the uniform parts go into the SGPR offset operand).
struct LoadOffsets {
    uint32_t a;      // A tile: 16 * lane
    uint32_t m;      // metadata: 4 * (lane & 31) + (lane >> 5) * tiles * 128 (second tile of the pair)
    uint32_t b[4];   // B row pair: (lane >> 5) * row pitch + 16 * swizzled chunk, by row & 3 >> 1 and row >> 3 & 1
};

__device__ __forceinline__ LoadOffsets load_offsets(const Args& a, int lane) {
    LoadOffsets o;
    const int tiles = (int)(a.K / BK);
    o.a = 16 * lane;
    o.m = 4 * (lane & 31) + (lane >> 5) * tiles * 128;
    const int pc = lane & 31;  // 16-byte slot in the LDS row
#pragma unroll
    for (int h = 0; h < 4; h++) {
        // a row with the same (row & 3) and (row >> 3) & 1 as this lane's row of the pair
        const int row = 2 * (h & 1) + (lane >> 5) + 8 * (h >> 1);
        const int v = ((row & 3) << 1) | ((row >> 3) & 1);
        const int lc = pc ^ (2 * v);  // 16-byte chunk of the X row
        o.b[h] = (uint32_t)((lane >> 5) * a.ldx * 2 + 16 * lc);
    }
    return o;
}

// Issue this wave's share of the loads of stage `s` into the stage buffer at LDS address `lds`.
// rA / rM cover the compressed tiles of this workgroup's row blocks (at most 16; tile (b, s) of block
// b at (b * tiles + s) * 1 KB of values and * 128 B of metadata). For s >= S (the pipeline runs three
// stages ahead and issues these unconditionally) the offsets get bit 31 set, past every record
// count, so the loads return zeros without memory traffic; rB's record count is 0 there anyway.
__device__ __forceinline__ void load_stage(uint32_t lds, const Args& a, i32x4 rA, i32x4 rM, int64_t n0, int s, int S,
                                           int wave, const LoadOffsets& lo) {
    const int64_t k0 = (int64_t)s * BK;
    const int tiles = (int)(a.K / BK);
    const uint32_t past = s < S ? 0u : 0x80000000u;
    // A: one 1 KB tile per 16-row block, copied as is (it is already in lane order)
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int b = 4 * wave + j;
        dma16(lds + b * 1024, lo.a + (((uint32_t)(b * tiles + s) * 1024u) | past), rA);
    }
    // metadata: one 128 B tile per block; 4 blocks per wave, two per dword instruction
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int b = 4 * wave + 2 * h;
        dma4(lds + A_BYTES + b * 128, lo.m + (((uint32_t)(b * tiles + s) * 128u) | past), rM);
    }
    // B: 64 rows x 512 B; this wave loads rows 16*wave .. +15, two rows per instruction (rows
    // 16 wave + 2h + lane / 32: row & 3 = 2 (h & 1) + lane / 32, (row >> 3) & 1 = h >> 2).
    // X's exact extent from this stage's corner ((K - 1) rows of pitch ldx plus N elements); make_rsrc
    // rounds it up to whole dwords (the range check passes a dword only if all of it is in range)
    const i32x4 rB = make_rsrc(a.X + k0 * a.ldx + n0, ((a.K - 1 - k0) * a.ldx + a.N - n0) * 2);
#pragma unroll
    for (int h = 0; h < 8; h++) {
        const int row = 16 * wave + 2 * h;
        dma16(lds + A_BYTES + META_BYTES + row * B_ROW,
              lo.b[(h & 1) | ((h >> 2) << 1)] + (uint32_t)(row * a.ldx * 2), rB);
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
    // read t of group q covers rows 8q + 4(t&1) + 32(t>>1) + r/4, which all have the row & 3 and
    // (row >> 3) & 1 of row0, so the unit swizzle is fixed per lane and t only adds immediates
    const int row0 = 8 * q + (r >> 2);
    const int v = ((row0 & 3) << 1) | ((row0 >> 3) & 1);
#pragma unroll
    for (int j = 0; j < FN; j++) {
        const int col = wn0 + 16 * j + 4 * (r & 3);  // first of the 4 columns this lane points at
        o.b[j] = A_BYTES + META_BYTES + row0 * B_ROW + (((col >> 4) ^ v) << 5) + 2 * (col & 15);
    }
    return o;
}

// Operands of one stage held in registers: the 8 A fragments and their indices.
struct AFrags {
    bf16x8 a[FM];
    uint32_t idx[FM];
};

typedef __attribute__((address_space(3))) char lds_char;

// A lane's LDS address for this stage's buffer, made opaque to the optimizer: otherwise it hoists
// the (lane offset + immediate) sums of every read out of the K loop, 32 loop-invariant registers
// for B alone, instead of folding the immediates into the reads' offset fields.
__device__ __forceinline__ uint32_t stage_addr(uint32_t buf, int off) {
    uint32_t v = buf + (uint32_t)off;
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ void read_a(uint32_t buf, const LaneOffsets& o, AFrags& f) {
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(buf, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(buf, o.m);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        f.a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
        f.idx[i] = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(pm + i * 128);
    }
}

// B fragment j (16 columns x 64 k) of the stage in buffer `buf`: four transposing reads.
__device__ __forceinline__ bf16x16 read_b(uint32_t buf, const LaneOffsets& o, int j) {
    const lds_char* p = (const lds_char*)(size_t)stage_addr(buf, o.b[j]);
    u32x8 b;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        // t = 0, 1: rows 8q + 4t + r/4; t = 2, 3: the same + 32
        const int imm = (t & 1) * 4 * B_ROW + (t >> 1) * 32 * B_ROW;
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + imm));
        b[2 * t] = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
        b[2 * t + 1] = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    }
    return __builtin_bit_cast(bf16x16, b);
}

__device__ __forceinline__ void mfma_block(f32x4 (&acc)[FM][FN], const AFrags& f, const bf16x16& b, int j) {
#pragma unroll
    for (int i = 0; i < FM; i++)
        acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(f.a[i], b, acc[i][j], (int)f.idx[i], 0, 0);
}

// One K stage (see the pipeline description in the kernel). The body has no branches: past the
// last stage the loads are out of range and the reads of the "next" buffer are never used.
__device__ __forceinline__ void stage(uint32_t l0, const Args& a, i32x4 rA, i32x4 rM, int64_t n0, int s, int S,
                                      f32x4 (&acc)[FM][FN], AFrags& f, bf16x16 (&rb)[4], const LaneOffsets& o,
                                      int wave, const LoadOffsets& lo) {
    const int cb = s % 3;
    const uint32_t cur = l0 + cb * STAGE_BYTES;
    const uint32_t nxt = l0 + (cb == 2 ? 0 : cb + 1) * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < 6; j++) {
        rb[(j + 2) & 3] = read_b(cur, o, j + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, f, rb[j & 3], j);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage s are done
    wait_vmcnt<LOADS_PER_STAGE>();       // stage s+1 has landed (s+2 may still be in flight)
    __builtin_amdgcn_s_barrier();
    load_stage(cur, a, rA, rM, n0, s + 3, S, wave, lo);
    rb[0] = read_b(nxt, o, 0);
    rb[1] = read_b(nxt, o, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(acc, f, rb[2], 6);
    __builtin_amdgcn_sched_barrier(0);
    // last block: once fragment i has been used for the last time, reload it (and its index) from the
    // next stage, so one A register set serves the whole pipeline
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(nxt, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(nxt, o.m);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][7] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(f.a[i], rb[3], acc[i][7], (int)f.idx[i], 0, 0);
        f.a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
        f.idx[i] = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(pm + i * 128);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------- epilogues
// The accumulators hold, per lane, 4 consecutive rows of one column; Y wants runs along a row. Each
// wave stages its 128 x 128 tile through LDS (reusing the pipeline buffers) so global stores are
// 16 bytes per lane with 64 contiguous bytes per row segment.

// bf16: the tile is written column-major (one column = 128 rows, pitch EPI_COL bytes, padded so
// both the 8-byte writes and the transposing reads below are free of bank conflicts), then read back
// with ds_read_b64_tr_b16, which hands each lane 4 consecutive columns of one row.
constexpr int EPI_COL = 128 * 2 + 40;
static_assert(4 * 128 * EPI_COL <= 3 * STAGE_BYTES, "epilogue staging fits in the stage buffers");

__device__ __forceinline__ void store_bf16(char* smem, const f32x4 (&acc)[FM][FN], const Args& a, int64_t mw, int64_t nw,
                                           int wave, int lane) {
    const int r = lane & 15, q = lane >> 4;
    char* tile = smem + wave * 128 * EPI_COL;
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const uint32_t lo = f32_to_bf16_rne(acc[i][j][0]) | ((uint32_t)f32_to_bf16_rne(acc[i][j][1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(acc[i][j][2]) | ((uint32_t)f32_to_bf16_rne(acc[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(tile + (16 * j + r) * EPI_COL + (16 * i + 4 * q) * 2) = make_uint2(lo, hi);
        }
        __builtin_amdgcn_sched_barrier(0);  // convert row block by row block (bounded live registers)
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    // 32 steps of 16 rows x 32 columns: group q takes columns cb + 8q .. +7 of rows rb .. rb+15
    const bool full = (mw + 128 <= a.M) && (nw + 128 <= a.N);
#pragma unroll
    for (int rb = 0; rb < 128; rb += 16)
#pragma unroll
        for (int cb = 0; cb < 128; cb += 32) {
            const int c0 = cb + 8 * q;
            // lane s of the group points at column c0 + s/4 (+4), rows rb + 4(s%4) .. +3
            const char* p0 = tile + (c0 + (r >> 2)) * EPI_COL + (rb + 4 * (r & 3)) * 2;
            const i16x4 u = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(p0 + 4 * EPI_COL));
            const int64_t m = mw + rb + r, n = nw + c0;
            const uint4 val = make_uint4((uint16_t)u[0] | ((uint32_t)(uint16_t)u[1] << 16),
                                         (uint16_t)u[2] | ((uint32_t)(uint16_t)u[3] << 16),
                                         (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16),
                                         (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16));
            uint16_t* y = reinterpret_cast<uint16_t*>(a.Y) + m * a.ldy + n;
            if (full && a.y_vec) {
                *reinterpret_cast<uint4*>(y) = val;
            } else if (m < a.M) {
                const uint16_t e[8] = {(uint16_t)val.x, (uint16_t)(val.x >> 16), (uint16_t)val.y, (uint16_t)(val.y >> 16),
                                       (uint16_t)val.z, (uint16_t)(val.z >> 16), (uint16_t)val.w, (uint16_t)(val.w >> 16)};
#pragma unroll
                for (int k = 0; k < 8; k++)
                    if (n + k < a.N) y[k] = e[k];
            }
        }
}

// fp32: two passes of 64 rows; the half-tile is written row-major (pitch EPI_ROW32 bytes, padded)
// with one 4-byte write per value and read back 16 bytes (4 columns) per lane.
constexpr int EPI_ROW32 = 128 * 4 + 16;
static_assert(4 * 64 * EPI_ROW32 <= 3 * STAGE_BYTES, "epilogue staging fits in the stage buffers");

__device__ __forceinline__ void store_fp32(char* smem, const f32x4 (&acc)[FM][FN], const Args& a, int64_t mw, int64_t nw,
                                           int wave, int lane) {
    const int r = lane & 15, q = lane >> 4;
    char* tile = smem + wave * 64 * EPI_ROW32;
    const bool full = (mw + 128 <= a.M) && (nw + 128 <= a.N);
#pragma unroll
    for (int half = 0; half < 2; half++) {
#pragma unroll
        for (int i = 0; i < FM / 2; i++) {
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int t = 0; t < 4; t++)
                    *reinterpret_cast<float*>(tile + (16 * i + 4 * q + t) * EPI_ROW32 + (16 * j + r) * 4) =
                        acc[half * (FM / 2) + i][j][t];
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        // 64 rows x 128 columns: each step covers 2 rows (32 lanes x 4 columns per row)
#pragma unroll
        for (int rr = 0; rr < 64; rr += 2) {
            const int row = rr + (lane >> 5), col = 4 * (lane & 31);
            const float4 v = *reinterpret_cast<const float4*>(tile + row * EPI_ROW32 + col * 4);
            const int64_t m = mw + 64 * half + row, n = nw + col;
            float* y = reinterpret_cast<float*>(a.Y) + m * a.ldy + n;
            if (full && a.y_vec) {
                *reinterpret_cast<float4*>(y) = v;
            } else if (m < a.M) {
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; k++)
                    if (n + k < a.N) y[k] = e[k];
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
}

template <bool OUT_FP32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_tiled_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) char smem[3 * STAGE_BYTES];
    // LDS byte addresses of the three stage buffers (for the LDS-destination loads)
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    const uint32_t l1 = l0 + STAGE_BYTES, l2 = l0 + 2 * STAGE_BYTES;

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

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    // compressed tiles of this workgroup's first row block onward (rows are padded to 16)
    const int64_t tiles = a.K / BK, blocks_left = (a.M + 15) / 16 - m0 / 16;
    const int64_t blocks = blocks_left < BM / 16 ? blocks_left : BM / 16;
    const i32x4 rA = make_rsrc(reinterpret_cast<const char*>(a.vals) + (m0 / 16) * tiles * 1024, blocks * tiles * 1024);
    const i32x4 rM = make_rsrc(a.meta + (m0 / 16) * tiles * 128, blocks * tiles * 128);

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const LaneOffsets o = lane_offsets(wm0, wn0, lane);
    const LoadOffsets lo = load_offsets(a, lane);
    const int S = (int)(a.K / BK);

    // Software pipeline over K stages of 64 columns, three LDS buffers (stage s in buffer s % 3):
    //  - the loads of stage s+3 go out once every wave has finished reading stage s, i.e. at the
    //    barrier placed before the last two fragment blocks of stage s, so each stage's loads have
    //    about two stages of compute to land;
    //  - that barrier also publishes stage s+1 (each wave first waits for its own loads of it), so
    //    stage s+1's A fragments, indices and first B fragments are read while the last 16
    //    smfmacs of stage s run;
    //  - inside a stage, B fragment j+2 is read while fragment j is multiplied (ring of 4).
    load_stage(l0, a, rA, rM, n0, 0, S, wave, lo);
    load_stage(l1, a, rA, rM, n0, 1, S, wave, lo);
    wait_vmcnt<LOADS_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    load_stage(l2, a, rA, rM, n0, 2, S, wave, lo);

    AFrags fa;
    bf16x16 rb[4];
    read_a(l0, o, fa);
    rb[0] = read_b(l0, o, 0);
    rb[1] = read_b(l0, o, 1);
    for (int s = 0; s < S; s++) stage(l0, a, rA, rM, n0, s, S, acc, fa, rb, o, wave, lo);

    // epilogue: lane holds column n0 + wn0 + 16 j + r, rows m0 + wm0 + 16 i + 4 q + t
    wait_vmcnt<0>();               // the zero-filling loads past the last stage have landed
    __builtin_amdgcn_s_barrier();  // every wave is done reading (and loading) the stage buffers
    if (OUT_FP32)
        store_fp32(smem, acc, a, m0 + wm0, n0 + wn0, wave, lane);
    else
        store_bf16(smem, acc, a, m0 + wm0, n0 + wn0, wave, lane);
}

}  // namespace tiled_bf16

bool gemm_bf16_tiled_ok(int64_t M, int64_t K, int64_t N, int64_t ldx, const void* X) {
    // 32-bit load offsets: 64 rows of X (64 * ldx * 2 < 2^31) and 16 row blocks of compressed tiles
    // (16 * K / 64 * 1 KB < 2^31) stay below bit 31, which marks the loads past the last stage
    return K % tiled_bf16::BK == 0 && ldx % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0 && N > 64 &&
           ldx < ((int64_t)1 << 24) && K < ((int64_t)1 << 22) && ((M + 255) / 256) * ((N + 255) / 256) < (1 << 30);
}

hipError_t launch_gemm_bf16_tiled(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                                  int64_t N, int64_t ldx, void* Y, bool out_fp32, int64_t ldy, hipStream_t s) {
    tiled_bf16::Args a;
    a.vals = values; a.meta = meta; a.X = X; a.Y = Y;
    a.M = M; a.K = K; a.N = N; a.ldx = ldx; a.ldy = ldy;
    a.tilesM = (int)((M + tiled_bf16::BM - 1) / tiled_bf16::BM);
    a.tilesN = (int)((N + tiled_bf16::BN - 1) / tiled_bf16::BN);
    a.y_vec = ((reinterpret_cast<uintptr_t>(Y) & 15) == 0) && ((ldy * (out_fp32 ? 4 : 2)) % 16 == 0);
    const unsigned grid = (unsigned)(a.tilesM * a.tilesN);
    if (out_fp32)
        hipLaunchKernelGGL(tiled_bf16::gemm_bf16_tiled_kernel<true>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(tiled_bf16::gemm_bf16_tiled_kernel<false>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sp24
