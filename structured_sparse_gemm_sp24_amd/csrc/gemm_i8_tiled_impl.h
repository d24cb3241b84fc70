// Tiled sparse x dense GEMM for large N, int8 in, exact int32 accumulation, per-output-channel fp32
// dequant epilogue (oeforum post on sparse acceleration: int8 and 2:4 combine; Orin NN design,
// Chapter 7, section 3.1 Step 4; NVIDIA blog on Ampere structured sparsity, Figure 1).
//
// Same organisation as the bf16 tiled kernel, with v_smfmac_i32_16x16x128_i8:
// workgroup tile 256 (M) x 256 (N), 4 waves in a 2 x 2 grid, each wave 128 x 128 = 8 x 8 fragments
// (256 int32 accumulators per lane, one wave per SIMD). K advances 128 dense columns per stage; three
// stages are in flight through LDS (3 x 52 KB):
//   A (compressed values): one 1 KB tile per 16-row block, already in the operand's lane order
//     (lane l holds 16 kept int8 of row l % 16, dense columns [32 (l / 16), +32));
//   metadata: one 256 B tile per block (lane l's 32-bit index at 4 l);
//   B tile (X, 128 rows x 256 int8 = 256 B per row): row-major with the 16-byte units of row k
//     stored at unit ^ f(k), f(k) = (k & 7) + 8 ((k >> 4) & 1). One ds_read_b64_tr_b8 takes 8 rows x
//     16 bytes per 16-lane group, rows 16q + {0..7} (+8, +64) for q = 0..3; f puts those 32 rows in 16
//     distinct 16-byte bank slots (two rows each, the minimum for 512 bytes), and stays the same for
//     the +8 / +64 row offsets, so those are immediates. Every 4 consecutive lanes of a global load
//     still read one aligned 64-byte run.
// The B operand (lane = column, 32 k values: k = 16q + (e & 15) + 64 (e >> 4)) comes from four
// ds_read_b64_tr_b8: in each 16-lane group, lane s points at row k0 + s/2, columns c0 + 8 (s % 2);
// the instruction hands lane i the 8 consecutive k of column c0 + i.
//
// Loads are buffer loads with LDS destination whose whole byte offset is in the range-checked VGPR
// operand: reads past this workgroup's row blocks, past K and past the end of X return zeros, and the
// loads the pipeline issues past the workgroup's last tile are pushed out of range on purpose.
// Persistent like the bf16 kernel: one workgroup per CU (two for token-major 128-wide tiles, see Cfg)
// walks its tiles (neighbouring tiles on the same XCD at the same time, groups of 8 tile-rows) with the
// LDS pipeline continued across tiles; the epilogue dequantizes in registers, transposes 4 x 4 blocks
// inside lane quads by DPP and stores 16 bytes per lane, so its stores drain while the next tile
// computes.
//
// Token-major X (N x K) and Y (N x M): the B tile is 256 token rows x 128 k (128 B per row), a lane's
// operand two 16-byte runs of its token's row (k = 16q .. +15 and 64 + 16q .. +15), read with two
// ds_read_b128 from units stored at unit ^ f(n), f(n) = ((n >> 1) & 7) ^ 4 (n & 1) (conflict-free, as
// in the bf16 kernel); each accumulator's 4 consecutive rows of M are one 16-byte store of token row
// n. K must be a multiple of 128 there. A batch of products sharing the weight adds the batch to the
// tile index.
#pragma once
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace tiled_i8 {

constexpr int BM = 256, BK = 128;
constexpr int WM = 128;
constexpr int FM = WM / 16;
constexpr int A_BYTES = BM * 64;          // 64 kept int8 per row per stage
constexpr int META_BYTES = BM * 16;       // 64 kept values x 2 bits = 16 bytes per row
constexpr int GROUP_M = 8;
constexpr uint32_t RSRC_FLAGS = 0x00020000u;

// Tile width BN: 256 (waves of 128 x 128, three 52 KB stage buffers), or 128 (waves of 128 x 64, four
// 36 KB buffers), chosen per launch (tiled_tile_width). A feature-major B tile row is BN bytes.
// PAIR (token-major, BN = 128 only): two workgroups per compute unit, each with two stage buffers and
// at most 256 registers per lane, so that one workgroup's epilogue (VALU work and the tile's store burst)
// runs beside the other's main loop instead of leaving the matrix cores idle.
template <int BN_, bool PAIR_ = false>
struct Cfg {
    static constexpr int BN = BN_, WN = BN_ / 2, FN = WN / 16;
    static constexpr bool PAIR = PAIR_;
    static constexpr int B_BYTES = BK * BN;  // token-major: BN rows x 128 B; feature-major: 128 rows x BN B
    static constexpr int STAGE_BYTES = A_BYTES + META_BYTES + B_BYTES;
    static constexpr int NBUF = PAIR ? 2 : (BN == 256 ? 3 : 4);
    static constexpr int B_LOADS = BN / 32;  // per wave
    static constexpr int LOADS_PER_STAGE = 4 + 1 + B_LOADS;  // per wave: A, metadata, B
    static_assert(!PAIR || BN == 128, "two workgroups per compute unit only with 128-wide tiles");
    static_assert((PAIR ? 2 : 1) * NBUF * STAGE_BYTES <= 160 * 1024, "the stage buffers fit in LDS");
};

// Raw buffer descriptor over `bytes` bytes rounded up to whole dwords: the range check returns a
// dword only when all of it is below the record count, and the rounding keeps the last partial dword
// of the real data (that dword lies in the same page as the data it ends).
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

// Buffer load with LDS destination (lane i's 16 bytes land at lds + 16 i), from inline asm so the
// compiler adds no waits of its own; ordered by explicit s_waitcnt vmcnt + s_barrier. No VGPR is
// written. `lds` is wave-uniform; `voff` is the lane's whole byte offset (range-checked).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct Args {
    const int8_t* vals;
    const uint8_t* meta;
    const int8_t* X;
    const float* scale;
    const float* bias;
    void* Y;
    int64_t M, K, N, ldx, ldy;
    float inv_scale;  // fl32(1 / out_scale) of int8 output
    int gelu;
    int64_t sxb, syb;  // batch strides (elements)
    int tilesM, tilesN, batch;
    int es;  // output element size
    int y_vec;  // Y base and row pitch allow 16-byte stores, 4 rows < 2^31 bytes
};

// Corner and compressed-tile descriptors of one tile; `valid` is false past the workgroup's last tile.
struct TileDesc {
    int64_t m0, n0;
    const int8_t* x;  // X and Y of the tile's batch entry
    char* y;
    i32x4 rA, rM;
    bool valid;
};

// Logical tile of workgroup p at its k-th turn, or -1. Turn k covers tiles [kG, kG + rem), rem =
// min(G, T - kG), split evenly over the 8 XCDs (workgroup p runs on XCD p % 8): XCD x takes a
// contiguous run of rem / 8 or rem / 8 + 1 of them, so a partial last turn still spreads its tiles,
// and their output writes, over every XCD, and neighbouring tiles share an L2.
__device__ __forceinline__ int tile_of(const Args& a, int p, int k) {
    const int G = gridDim.x, T = a.tilesM * a.tilesN * a.batch;
    const int64_t base = (int64_t)k * G;
    if (base >= T) return -1;
    const int rem = (T - base) < G ? (int)(T - base) : G;
    const int x = p & 7, i = p >> 3, q8 = rem >> 3, r8 = rem & 7;
    if (i >= q8 + (x < r8 ? 1 : 0)) return -1;
    return (int)base + x * q8 + (x < r8 ? x : r8) + i;
}

// Swizzle of the 16-byte units of B row k (see the header).
__device__ __forceinline__ int bswz(int k) { return (k & 7) | (((k >> 4) & 1) << 3); }
// The same for the 128-byte rows of the 128-wide feature-major tile (8 units): g(k) = ((k >> 1) & 3) +
// 4 ((k >> 4) & 1). A read's rows 16q + {0..7} then take bank slots 8 (k & 1) + (u ^ g(k)): groups q and
// q + 1 together fill all 16 slots once, so each slot serves two rows (the minimum for 512 bytes); g is
// unchanged by the +8 / +64 row offsets of the reads, and XOR with g keeps each 4-lane group of a
// global load on one aligned 64-byte run.
__device__ __forceinline__ int bswz128(int k) { return ((k >> 1) & 3) | (((k >> 4) & 1) << 2); }

// 16-byte unit swizzle of token row n of a token-major B tile.
__device__ __forceinline__ int tm_swz(int n) { return ((n >> 1) & 7) ^ ((n & 1) << 2); }

// Per-lane parts of the load offsets.
struct LoadOffsets {
    uint32_t a;      // A tile: 16 * lane
    uint32_t m;      // metadata: tile (lane / 16) of the wave's 4 blocks, 16 * (lane % 16) inside it
    uint32_t b[8];   // B rows 4h + lane / 16 of the wave's 32 rows: row part + swizzled chunk;
                     // token-major: rows 8h + lane / 8 of the wave's 64 (row part relative to the wave's first)
};

template <bool TM, int BNT>
__device__ __forceinline__ LoadOffsets load_offsets(const Args& a, int lane, int wave) {
    LoadOffsets o;
    const int tiles = (int)((a.K + BK - 1) / BK);
    o.a = 16 * lane;
    o.m = (uint32_t)((lane >> 4) * tiles * 256 + 16 * (lane & 15));
    if constexpr (TM) {
        // lane i of a load lands in token row 8h + i / 8 of the wave's rows, 16-byte slot i % 8, and
        // reads the unit that belongs there
#pragma unroll
        for (int h = 0; h < 8; h++) {
            const int row = 8 * h + (lane >> 3);
            o.b[h] = (uint32_t)(row * a.ldx + 16 * ((lane & 7) ^ tm_swz(row)));
        }
        (void)wave;
    } else if constexpr (BNT == 256) {
        const int p = lane & 15;  // 16-byte slot in the LDS row
#pragma unroll
        for (int h = 0; h < 8; h++) {
            const int row = 32 * wave + 4 * h + (lane >> 4);
            o.b[h] = (uint32_t)(row * a.ldx + 16 * (p ^ bswz(row)));
        }
    } else {
        // 128-byte rows: lane i of load h lands in row 32 wave + 8h + i / 8, slot i % 8
        const int p = lane & 7;
#pragma unroll
        for (int h = 0; h < 4; h++) {
            const int row = 32 * wave + 8 * h + (lane >> 3);
            o.b[h] = (uint32_t)(row * a.ldx + 16 * (p ^ bswz128(row)));
        }
#pragma unroll
        for (int h = 4; h < 8; h++) o.b[h] = 0;
    }
    return o;
}

// This wave's share of the loads of stage s of tile td into the buffer at LDS address `lds`. When td
// is not valid the offsets get bit 31 set (beyond every record count): zeros, no memory traffic.
// The descriptor in scalar registers (the loads take it there): a no-op where the compiler already holds
// it there, a readfirstlane per word where register pressure made it keep the uniform words in VGPRs.
__device__ __forceinline__ i32x4 uniform_rsrc(const i32x4& r) {
    return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                 __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

template <bool TM, int BNT>
__device__ __forceinline__ void load_stage(uint32_t lds, const Args& a, const TileDesc& td, int s, int wave,
                                           const LoadOffsets& lo) {
    const int64_t k0 = (int64_t)s * BK;
    const int tiles = (int)((a.K + BK - 1) / BK);
    const uint32_t past = td.valid ? 0u : 0x80000000u;
    const i32x4 rA = uniform_rsrc(td.rA), rM = uniform_rsrc(td.rM);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int b = 4 * wave + j;
        dma16(lds + b * 1024, lo.a + (((uint32_t)(b * tiles + s) * 1024u) | past), rA);
    }
    // metadata of blocks 4 wave .. 4 wave + 3 (one 256 B tile each) in one instruction
    dma16(lds + A_BYTES + 4 * wave * 256, lo.m + (((uint32_t)(4 * wave * tiles + s) * 256u) | past), rM);
    if constexpr (TM) {
        // token rows BNT/4 * wave .. +BNT/4-1 of the tile, 8 per load; X's extent from the wave's first
        // row: rows past N read zeros (K is a multiple of 128: no stage reaches past K)
        const int64_t n1 = td.n0 + (BNT / 4) * wave;
        const i32x4 rB = make_rsrc(td.x + n1 * a.ldx + k0, td.valid ? (a.N - 1 - n1) * a.ldx + a.K - k0 : 0);
#pragma unroll
        for (int h = 0; h < Cfg<BNT>::B_LOADS; h++)
            dma16(lds + A_BYTES + META_BYTES + ((BNT / 4) * wave + 8 * h) * 128, lo.b[h], rB);
    } else {
        // X's exact extent from this stage's corner, rounded up to whole dwords (see make_rsrc)
        const i32x4 rB = make_rsrc(td.x + k0 * a.ldx + td.n0, td.valid ? (a.K - 1 - k0) * a.ldx + a.N - td.n0 : 0);
        // this wave's 32 rows: 4 per load with 256-byte rows, 8 per load with 128-byte rows
        constexpr int RPL = 1024 / BNT;
#pragma unroll
        for (int h = 0; h < 32 / RPL; h++) dma16(lds + A_BYTES + META_BYTES + (32 * wave + RPL * h) * BNT, lo.b[h], rB);
    }
}

// Descriptor of logical tile L (-1: none); batch entries follow each other, and inside one tiles are
// walked in groups of GROUP_M tile-rows.
template <int BNT>
__device__ __forceinline__ TileDesc tile_desc(const Args& a, int L) {
    TileDesc td;
    td.valid = L >= 0;
    const int per = a.tilesM * a.tilesN;
    const int bt = L >= 0 ? L / per : 0;
    const int Lc = L >= 0 ? L - bt * per : 0;
    td.x = a.X + bt * a.sxb;
    td.y = static_cast<char*>(a.Y) + bt * a.syb * a.es;
    const int gsize = GROUP_M * a.tilesN;
    const int g = Lc / gsize;
    const int first_m = g * GROUP_M;
    const int gm = (a.tilesM - first_m) < GROUP_M ? (a.tilesM - first_m) : GROUP_M;
    const int in_g = Lc - g * gsize;
    const int tm = first_m + in_g % gm, tn = in_g / gm;
    td.m0 = (int64_t)tm * BM;
    td.n0 = (int64_t)tn * BNT;
    const int64_t tiles = (a.K + BK - 1) / BK, blocks_left = (a.M + 15) / 16 - td.m0 / 16;
    const int64_t blocks = blocks_left < BM / 16 ? blocks_left : BM / 16;
    td.rA = make_rsrc(reinterpret_cast<const char*>(a.vals) + (td.m0 / 16) * tiles * 1024, blocks * tiles * 1024);
    td.rM = make_rsrc(a.meta + (td.m0 / 16) * tiles * 256, blocks * tiles * 256);
    return td;
}

template <int FNT>
struct LaneOffsets {
    int a;       // A fragment of block wm0/16: block * 1024 + lane * 16
    int m;       // metadata: A_BYTES + block * 256 + lane * 4
    int b[FNT];   // B fragment j, first read (t = 0); token-major: the two reads of fragment 0
};

template <bool TM, int FNT>
__device__ __forceinline__ LaneOffsets<FNT> lane_offsets(int wm0, int wn0, int lane) {
    const int r = lane & 15, q = lane >> 4;
    LaneOffsets<FNT> o;
    o.a = (wm0 >> 4) * 1024 + lane * 16;
    o.m = A_BYTES + (wm0 >> 4) * 256 + lane * 4;
    if constexpr (TM) {
        const int base = A_BYTES + META_BYTES + (wn0 + r) * 128, u = q ^ tm_swz(r);
        o.b[0] = base + 16 * u;
        o.b[1] = base + 16 * (u ^ 4);
#pragma unroll
        for (int j = 2; j < FNT; j++) o.b[j] = 0;
        return o;
    }
    // read t of group q covers rows 16q + 8(t&1) + 64(t>>1) + r/2, which share row & 7 and
    // (row >> 4) & 1 with row0, so the swizzle is fixed per lane and t only adds immediates
    constexpr int B_ROW = 32 * FNT;  // the tile width in bytes
    const int row0 = 16 * q + (r >> 1);
    const int f = B_ROW == 256 ? bswz(row0) : bswz128(row0);
#pragma unroll
    for (int j = 0; j < FNT; j++) {
        const int unit = (wn0 >> 4) + j;  // 16 columns = one 16-byte unit
        o.b[j] = A_BYTES + META_BYTES + row0 * B_ROW + ((unit ^ f) << 4) + 8 * (r & 1);
    }
    return o;
}

struct AFrags {
    i32x4 a[FM];
    uint32_t idx[FM];
};

typedef __attribute__((address_space(3))) char lds_char;

// A lane's LDS address in this stage's buffer, opaque to the optimizer (keeps the immediates in the
// reads instead of dozens of hoisted loop-invariant sums).
__device__ __forceinline__ uint32_t stage_addr(uint32_t buf, int off) {
    uint32_t v = buf + (uint32_t)off;
    asm volatile("" : "+v"(v));
    return v;
}

template <int FNT>
__device__ __forceinline__ void read_a(uint32_t buf, const LaneOffsets<FNT>& o, AFrags& f) {
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(buf, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(buf, o.m);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(pa + i * 1024);
        f.idx[i] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(pm + i * 256);
    }
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// B fragment j (16 columns x 128 k): four transposing reads of 8 k each, or, token-major, two 16-byte
// reads of the lane's token row.
template <bool TM, int FNT>
__device__ __forceinline__ i32x8 read_b(uint32_t buf, const LaneOffsets<FNT>& o, int j) {
    if constexpr (TM) {
        typedef const __attribute__((address_space(3))) i32x4 lds_i32x4;
        const lds_char* p0 = (const lds_char*)(size_t)stage_addr(buf, o.b[0]);
        const lds_char* p1 = (const lds_char*)(size_t)stage_addr(buf, o.b[1]);
        const i32x4 lo = *reinterpret_cast<lds_i32x4*>(p0 + j * 2048);
        const i32x4 hi = *reinterpret_cast<lds_i32x4*>(p1 + j * 2048);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    constexpr int B_ROW = 32 * FNT;
    const lds_char* p = (const lds_char*)(size_t)stage_addr(buf, o.b[j]);
    i32x8 b;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int imm = ((t & 1) * 8 + (t >> 1) * 64) * B_ROW;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p + imm));
        b[2 * t] = v[0];
        b[2 * t + 1] = v[1];
    }
    return b;
}

template <int FNT>
__device__ __forceinline__ void mfma_block(i32x4 (&acc)[FM][FNT], const AFrags& f, const i32x8& b, int j) {
#pragma unroll
    for (int i = 0; i < FM; i++)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(f.a[i], b, acc[i][j], (int)f.idx[i], 0, 0);
}

// One K stage: stage s of the current tile, the workgroup's g-th stage (selects the buffer). B
// fragments are read two blocks ahead (ring of 4); before the last two blocks the barrier publishes
// stage g+1 and the loads of stage s+NBUF of this tile (or s+NBUF-S of the next) go into this buffer; the
// next stage's A fragments are reloaded one by one inside the last block. No branches. NEXT = false
// (a tile's last stage with two workgroups per compute unit) leaves the next stage's operands unread,
// so they do not occupy registers through the epilogue; the kernel reads them after it.
template <bool TM, int BNT, bool PAIR, bool NEXT>
__device__ __forceinline__ void stage(uint32_t l0, const Args& a, const TileDesc& cur_t, const TileDesc& next_t, int s,
                                      int S, int g, i32x4 (&acc)[FM][Cfg<BNT>::FN], AFrags& f, i32x8 (&rb)[4],
                                      const LaneOffsets<Cfg<BNT>::FN>& o, int wave, const LoadOffsets& lo) {
    using C = Cfg<BNT, PAIR>;
    constexpr int F = C::FN, NB = C::NBUF;
    const int cb = g % NB;
    const uint32_t cur = l0 + cb * C::STAGE_BYTES;
    const uint32_t nxt = l0 + (cb == NB - 1 ? 0 : cb + 1) * C::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < F - 2; j++) {
        rb[(j + 2) & 3] = read_b<TM>(cur, o, j + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, f, rb[j & 3], j);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's reads of stage g are done
    wait_vmcnt<(NB - 2) * C::LOADS_PER_STAGE>();  // stage g+1 has landed
    __builtin_amdgcn_s_barrier();
    const bool here = s + NB < S;
    load_stage<TM, BNT>(cur, a, here ? cur_t : next_t, here ? s + NB : s + NB - S, wave, lo);
    if constexpr (!NEXT) {
        mfma_block(acc, f, rb[(F - 2) & 3], F - 2);
        mfma_block(acc, f, rb[(F - 1) & 3], F - 1);
        return;
    }
    rb[0] = read_b<TM>(nxt, o, 0);
    rb[1] = read_b<TM>(nxt, o, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(acc, f, rb[(F - 2) & 3], F - 2);
    __builtin_amdgcn_sched_barrier(0);
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(nxt, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(nxt, o.m);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][F - 1] =
            __builtin_amdgcn_smfmac_i32_16x16x128_i8(f.a[i], rb[(F - 1) & 3], acc[i][F - 1], (int)f.idx[i], 0, 0);
        f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(pa + i * 1024);
        f.idx[i] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(pm + i * 256);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Epilogue from registers, four fragments (64 columns) at a time. Each accumulator goes through the
// value pipeline (raw int32; or dequant fl32(fl32(acc) * scale[m]), optional bias and GELU) and is
// converted to the output type (int32/fp32 words, bf16 pairs rounded to nearest even, int8 codes
// clamp(rne(y / out_scale))). Then, as in the bf16 kernel, the quad transposes of each fragment and a
// quad transpose across the four fragments give lane (q, 4a + x) row 4q + s, columns 16x + 4a .. +3 in
// slot s, so a lane quad stores into one row (one request per 128-byte line instead of one per lane),
// and each store instruction writes 4 rows x 64 columns -- whole 128-byte lines except for int8
// output, whose two 64-byte halves of a line follow each other. No LDS is used.
template <int OUT>
struct OutTraits {
    static constexpr int ES = OUT == OUT_BF16 ? 2 : (OUT == OUT_I8 ? 1 : 4);  // element bytes
    static constexpr int W = OUT == OUT_BF16 ? 2 : (OUT == OUT_I8 ? 1 : 4);   // words per 4 elements
};

// Element k (0..3) of a lane's 4-element group, as the output type's bits.
template <int OUT>
__device__ __forceinline__ uint32_t out_elem(const uint32_t* v, int k) {
    if constexpr (OUT == OUT_BF16) return (k & 1 ? v[k >> 1] >> 16 : v[k >> 1]) & 0xFFFFu;
    else if constexpr (OUT == OUT_I8) return (v[0] >> (8 * k)) & 0xFFu;
    else return v[k];
}

template <int OUT>
__device__ __forceinline__ void store_elem(char* y, int64_t idx, uint32_t bits) {
    if constexpr (OUT == OUT_BF16) reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bits;
    else if constexpr (OUT == OUT_I8) reinterpret_cast<uint8_t*>(y)[idx] = (uint8_t)bits;
    else reinterpret_cast<uint32_t*>(y)[idx] = bits;
}

// One lane's group of output elements, with the non-temporal hint (the output is not read again here;
// streaming it out shortens the drain after the last tiles: 768 x 3072 x 8192 fp32 out 26.3 -> 24.8 us).
template <int OUT>
__device__ __forceinline__ void store_group(char* p, const uint32_t* v) {
    if constexpr (OutTraits<OUT>::W == 4) __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<u32x4*>(p));
    else if constexpr (OutTraits<OUT>::W == 2) __builtin_nontemporal_store(u32x2{v[0], v[1]}, reinterpret_cast<u32x2*>(p));
    else __builtin_nontemporal_store(v[0], reinterpret_cast<uint32_t*>(p));
}

// The 4 accumulators of one lane and fragment (rows m .. m+3 of one column, or, token-major, 4
// consecutive elements of one token row) through the value pipeline into the output type's words:
// 4 words (int32/fp32), 2 packed bf16 pairs, or 1 word of 4 int8 codes (element t in byte t).
template <int OUT, int EPI>
__device__ __forceinline__ void to_out(const i32x4& c, const float (&sc)[4], const float (&bi)[4], const Args& a,
                                       uint32_t* w) {
    constexpr bool BIAS = (EPI & 1) != 0, GELU = (EPI & 2) != 0;
    if constexpr (OUT == OUT_I32) {
#pragma unroll
        for (int t = 0; t < 4; t++) w[t] = (uint32_t)c[t];
    } else {
        f32x4 y;
#pragma unroll
        for (int t = 0; t < 4; t++) y[t] = i8_dequant(c[t], sc[t], bi[t], BIAS);
        if constexpr (GELU) y = gelu4_f32(y);
        if constexpr (OUT == OUT_F32) {
#pragma unroll
            for (int t = 0; t < 4; t++) w[t] = __float_as_uint(y[t]);
        } else if constexpr (OUT == OUT_BF16) {
            w[0] = pack_bf16x2_rne(y[0], y[1]);
            w[1] = pack_bf16x2_rne(y[2], y[3]);
        } else {
            w[0] = quant_i8x4(y, a.inv_scale);
        }
    }
}

// Dequant scale and bias of output rows m .. m+3 (zero past M).
template <int OUT, int EPI>
__device__ __forceinline__ void row_params(const Args& a, int64_t m, bool full, float (&sc)[4], float (&bi)[4]) {
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const bool ok = OUT != OUT_I32 && (full || m + t < a.M);
        sc[t] = ok ? a.scale[m + t] : 0.f;
        bi[t] = (ok && (EPI & 1)) ? a.bias[m + t] : 0.f;
    }
}

// FULL: the wave's whole 128 x 128 block lies inside Y and vector stores are allowed (then the row
// offsets of a lane quad fit 32 bits); otherwise every element is bounds-checked.
template <int OUT, int EPI, bool FULL, int FNT>
__device__ __forceinline__ void store_tile(const i32x4 (&acc)[FM][FNT], const Args& a, char* y, int64_t mw, int64_t nw,
                                           int lane) {
    constexpr int ES = OutTraits<OUT>::ES, W = OutTraits<OUT>::W;
    const int q = lane >> 4, r = lane & 15, b = r & 3, a4 = r >> 2;
    const uint32_t sel = half_sel(b);
    char* const y0 = y + (mw * a.ldy + nw) * ES;  // wave-uniform corner
    // lane (q, 4 a4 + b) stores row 4q + s, columns 16 b + 4 a4 .. +3 of the 64-column group
    const uint32_t lane_off = FULL ? (uint32_t)((4 * q * a.ldy + 16 * b + 4 * a4) * ES) : 0u;
#pragma unroll
    for (int i = 0; i < FM; i++) {
        float sc[4], bi[4];
        row_params<OUT, EPI>(a, mw + 16 * i + 4 * q, FULL, sc, bi);  // accumulator rows 4q .. 4q+3
#pragma unroll
        for (int jg = 0; jg < FNT / 4; jg++) {
            uint32_t v[4][W];
#pragma unroll
            for (int f = 0; f < 4; f++) {
                if constexpr (OUT == OUT_BF16) {
                    f32x4 y;
#pragma unroll
                    for (int t = 0; t < 4; t++) y[t] = i8_dequant(acc[i][4 * jg + f][t], sc[t], bi[t], (EPI & 1) != 0);
                    if constexpr ((EPI & 2) != 0) y = gelu4_f32(y);
                    const float e[4] = {y[0], y[1], y[2], y[3]};
                    quad_transpose_bf16(e, v[f], b, sel);
                } else if constexpr (OUT == OUT_I8) {
                    uint32_t w[1];
                    to_out<OUT, EPI>(acc[i][4 * jg + f], sc, bi, a, w);
                    v[f][0] = quad_transpose_u8(w[0], b);
                } else {
                    to_out<OUT, EPI>(acc[i][4 * jg + f], sc, bi, a, v[f]);
                    quad_transpose(v[f], b);
                }
                if constexpr ((EPI & 2) != 0) __builtin_amdgcn_sched_barrier(0);  // one fragment's GELUs at a time
            }
            slot_transpose4<W>(v, b);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                if constexpr (FULL) {
                    store_group<OUT>(y0 + ((16 * i + s) * a.ldy + 64 * jg) * ES + lane_off, v[s]);
                } else {
                    const int64_t m = mw + 16 * i + 4 * q + s, n = nw + 64 * jg + 16 * b + 4 * a4;
                    if (m < a.M) {
#pragma unroll
                        for (int k = 0; k < 4; k++)
                            if (n + k < a.N) store_elem<OUT>(y, m * a.ldy + n + k, out_elem<OUT>(v[s], k));
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one row block of fragments at a time
    }
}

// Token-major epilogue: Y is N x M; each accumulator (column n, rows 4q .. 4q+3 of M) goes through the
// value pipeline and is 4 consecutive elements of token row n. As in the bf16 kernel, a quad transpose
// across four row fragments gives each lane quad one token row (elements 16x + 4q .. +3 of 64 M-columns
// in lane 4c + x), so each store instruction covers 16 token rows x 64 elements.
template <int OUT, int EPI, bool FULL, int FNT>
__device__ __forceinline__ void store_tile_tm(const i32x4 (&acc)[FM][FNT], const Args& a, char* y, int64_t mw,
                                              int64_t nw, int lane) {
    constexpr int ES = OutTraits<OUT>::ES, W = OutTraits<OUT>::W;
    const int q = lane >> 4, r = lane & 15, x = r & 3, c = r >> 2;
    char* const y0 = y + (nw * a.ldy + mw) * ES;  // wave-uniform corner
    const uint32_t lane_off = FULL ? (uint32_t)((4 * c * a.ldy + 16 * x + 4 * q) * ES) : 0u;
#pragma unroll
    for (int ig = 0; ig < FM / 4; ig++) {
        float sc[4][4], bi[4][4];
#pragma unroll
        for (int f = 0; f < 4; f++) row_params<OUT, EPI>(a, mw + 16 * (4 * ig + f) + 4 * q, FULL, sc[f], bi[f]);
#pragma unroll
        for (int j = 0; j < FNT; j++) {
            uint32_t v[4][W];
#pragma unroll
            for (int f = 0; f < 4; f++) {
                to_out<OUT, EPI>(acc[4 * ig + f][j], sc[f], bi[f], a, v[f]);
                if constexpr ((EPI & 2) != 0) __builtin_amdgcn_sched_barrier(0);  // one fragment's GELUs at a time
            }
            slot_transpose4<W>(v, x);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                if constexpr (FULL) {
                    store_group<OUT>(y0 + ((16 * j + s) * a.ldy + 64 * ig) * ES + lane_off, v[s]);
                } else {
                    const int64_t n = nw + 16 * j + 4 * c + s, m = mw + 64 * ig + 16 * x + 4 * q;
                    if (n < a.N) {
#pragma unroll
                        for (int t = 0; t < 4; t++)
                            if (m + t < a.M) store_elem<OUT>(y, n * a.ldy + m + t, out_elem<OUT>(v[s], t));
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int OUT, bool TM, int EPI, int BNT, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PAIR ? 2 : 1, PAIR ? 2 : 1)))
void gemm_i8_tiled_kernel(Args a) {
    using C = Cfg<BNT, PAIR>;
    constexpr int NB = C::NBUF, F = C::FN;
    __shared__ __attribute__((aligned(16))) char smem[NB * C::STAGE_BYTES];
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;

    const int p = blockIdx.x;
    const int L = tile_of(a, p, 0);
    if (L < 0) return;  // whole workgroup
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * C::WN;
    const LaneOffsets<F> o = lane_offsets<TM, F>(wm0, wn0, lane);
    const LoadOffsets lo = load_offsets<TM, BNT>(a, lane, wave);
    const int S = (int)((a.K + BK - 1) / BK);

    i32x4 acc[FM][F];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < F; j++) acc[i][j] = i32x4{0, 0, 0, 0};

    // NB-stage pipeline continued across the workgroup's tiles (see stage()); with fewer than NB
    // stages per tile every workgroup has one tile (see the launcher), so the prologue's loads past
    // the tile's stages (next_t invalid) only zero-fill
    TileDesc cur_t = tile_desc<BNT>(a, L);
    TileDesc next_t = tile_desc<BNT>(a, tile_of(a, p, 1));
#pragma unroll
    for (int i = 0; i < NB - 1; i++)
        load_stage<TM, BNT>(l0 + i * C::STAGE_BYTES, a, S > i ? cur_t : next_t, S > i ? i : 0, wave, lo);
    wait_vmcnt<(NB - 2) * C::LOADS_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    load_stage<TM, BNT>(l0 + (NB - 1) * C::STAGE_BYTES, a, S > NB - 1 ? cur_t : next_t, S > NB - 1 ? NB - 1 : 0, wave,
                        lo);

    AFrags fa;
    i32x8 rb[4];
    read_a(l0, o, fa);
    rb[0] = read_b<TM>(l0, o, 0);
    rb[1] = read_b<TM>(l0, o, 1);
    int g = 0;
    for (int k = 1;; k++) {
        if constexpr (PAIR) {
            for (int s = 0; s < S - 1; s++, g++)
                stage<TM, BNT, PAIR, true>(l0, a, cur_t, next_t, s, S, g, acc, fa, rb, o, wave, lo);
            stage<TM, BNT, PAIR, false>(l0, a, cur_t, next_t, S - 1, S, g, acc, fa, rb, o, wave, lo);
            g++;
        } else {
            for (int s = 0; s < S; s++, g++)
                stage<TM, BNT, PAIR, true>(l0, a, cur_t, next_t, s, S, g, acc, fa, rb, o, wave, lo);
        }
        {
            const int64_t mw = cur_t.m0 + wm0, nw = cur_t.n0 + wn0;
            const bool full = (mw + WM <= a.M) && (nw + C::WN <= a.N) && a.y_vec;
            if constexpr (TM) {
                if (full)
                    store_tile_tm<OUT, EPI, true>(acc, a, cur_t.y, mw, nw, lane);
                else
                    store_tile_tm<OUT, EPI, false>(acc, a, cur_t.y, mw, nw, lane);
            } else {
                if (full)
                    store_tile<OUT, EPI, true>(acc, a, cur_t.y, mw, nw, lane);
                else
                    store_tile<OUT, EPI, false>(acc, a, cur_t.y, mw, nw, lane);
            }
        }
        if (!next_t.valid) break;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < F; j++) acc[i][j] = i32x4{0, 0, 0, 0};
        cur_t = next_t;
        next_t = tile_desc<BNT>(a, tile_of(a, p, k + 1));
        if constexpr (PAIR) {
            // the next tile's first stage landed before the last stage's barrier, and its buffer is
            // refilled only after the next barrier
            const uint32_t buf = l0 + (g % NB) * C::STAGE_BYTES;
            read_a(buf, o, fa);
            rb[0] = read_b<TM>(buf, o, 0);
            rb[1] = read_b<TM>(buf, o, 1);
        }
    }
    wait_vmcnt<0>();  // the zero-filling loads past the last tile have landed before the workgroup ends
}

template <int OUT, bool TMV, int BNT, bool PAIR>
void launch_epi(int epi, dim3 grid, dim3 block, hipStream_t s, const Args& a) {
    switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_i8_tiled_kernel<OUT, TMV, 0, BNT, PAIR>), grid, block, 0, s, a); break;
    case 1: if constexpr (OUT != OUT_I32) hipLaunchKernelGGL((gemm_i8_tiled_kernel<OUT, TMV, 1, BNT, PAIR>), grid, block, 0, s, a); break;
    case 2: if constexpr (OUT != OUT_I32) hipLaunchKernelGGL((gemm_i8_tiled_kernel<OUT, TMV, 2, BNT, PAIR>), grid, block, 0, s, a); break;
    default: if constexpr (OUT != OUT_I32) hipLaunchKernelGGL((gemm_i8_tiled_kernel<OUT, TMV, 3, BNT, PAIR>), grid, block, 0, s, a); break;
    }
}

// Whether a token-major launch of T 128-wide tiles of S stages runs two workgroups per compute unit.
inline bool tiled_i8_pair(int T, int S, int cus) { return T > cus && S >= 2; }

// Launch for one output kind and tile width (instantiated in gemm_i8_tiled*.hip, one output kind per
// file so they compile in parallel): grid, arguments, and the layout x epilogue variant.
template <int OUT, int BNT>
hipError_t launch_bn(const GemmArgs& g, hipStream_t s) {
    using C = Cfg<BNT>;
    Args a;
    a.vals = static_cast<const int8_t*>(g.values); a.meta = g.meta;
    a.X = static_cast<const int8_t*>(g.X); a.scale = g.scale; a.bias = g.bias; a.Y = g.Y;
    a.M = g.M; a.K = g.K; a.N = g.N; a.ldx = g.ldx; a.ldy = g.ldy;
    a.inv_scale = g.inv_scale; a.gelu = g.gelu;
    a.sxb = g.sx; a.syb = g.sy;
    a.tilesM = (int)((g.M + BM - 1) / BM);
    a.tilesN = (int)((g.N + BNT - 1) / BNT);
    a.batch = (int)g.batch;
    constexpr int64_t es = OutTraits<OUT>::ES;
    a.es = (int)es;
    // vector stores: 16-byte aligned Y rows in every batch entry, and 16 rows' offsets in 32 bits
    a.y_vec = ((reinterpret_cast<uintptr_t>(g.Y) & 15) == 0) && ((g.ldy * es) % 16 == 0) &&
              (g.batch == 1 || (g.sy * es) % 16 == 0) && g.ldy * es * 16 < ((int64_t)1 << 31);
    const int T = a.tilesM * a.tilesN * a.batch;
    const int S = (int)((g.K + BK - 1) / BK);
    const int cus = device_cus();
    // the epilogue variant (bias, GELU) is a compile-time choice: GELU, and even a per-element bias
    // select, would otherwise cost every epilogue
    const int epi = OUT == OUT_I32 ? 0 : ((g.bias ? 1 : 0) | (g.gelu ? 2 : 0));
    const dim3 block(256);
    if constexpr (BNT == 128) {
        // two workgroups per compute unit when every one of them gets a tile and each has its two stages
        if (g.tm && tiled_i8_pair(T, S, cus)) {
            launch_epi<OUT, true, BNT, true>(epi, dim3((unsigned)(T > 2 * cus ? 2 * cus : T)), block, s, a);
            return hipGetLastError();
        }
    }
    // one workgroup per compute unit walking several tiles; one tile each when a tile has fewer stages
    // than there are stage buffers (the cross-tile pipeline then has nothing to overlap)
    const dim3 grid((unsigned)(S >= C::NBUF && T > cus ? cus : T));
    if (g.tm)
        launch_epi<OUT, true, BNT, false>(epi, grid, block, s, a);
    else
        launch_epi<OUT, false, BNT, false>(epi, grid, block, s, a);
    return hipGetLastError();
}

// Tile width: token-major products with at least two 128-wide tiles per compute unit take them, two
// workgroups per compute unit (faster than 256-wide tiles on every such shape measured: 4096^3 52.4 ->
// 49.7 us, 11008 x 4096 x 4096 146.5 -> 142.5, 3072 x 768 x 16384 58.9 -> 52.8, 8192^3 352 -> 349.5);
// the rest follow the turn-cost rule shared with the bf16 kernel.
template <int OUT>
hipError_t launch_out(const GemmArgs& g, hipStream_t s) {
    const int64_t t128 = ((g.M + BM - 1) / BM) * ((g.N + 127) / 128) * g.batch;
    if (g.tm && t128 >= 2 * (int64_t)device_cus() && g.K > BK) return launch_bn<OUT, 128>(g, s);
    return tiled_tile_width(g) == 128 ? launch_bn<OUT, 128>(g, s) : launch_bn<OUT, 256>(g, s);
}

}  // namespace tiled_i8
}  // namespace sp24
