// Tiled sparse x dense GEMM for large N, bf16 in, fp32 accumulate (NVIDIA blog on Ampere structured
// sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1 Step 3).
//
// Workgroup tile 256 (M) x BN (N); waves of 128 x WN hold 8 x WN/16 v_smfmac_f32_16x16x64_bf16 fragments.
// K advances 64 dense columns per stage through LDS stage buffers. Two main loops:
//  - token-major X (N x K, a Linear layer's input; gemm_bf16_tm_kernel): waves of 128 x 64, two per SIMD --
//    BN = 256 with eight waves and three 50 KB stage buffers, or BN = 128 with four waves, two 34 KB buffers
//    and two workgroups per compute unit. Its per-stage instruction stream is kept short (about 100
//    instructions per wave per stage, 32 of them smfmacs): buffer descriptors are made once per tile, the
//    lane part of every load offset once per kernel, and the stage's advance along K rides in the loads'
//    SGPR offset;
//  - feature-major X (K x N; gemm_bf16_tiled_kernel): BN = 256 with four waves of 128 x 128 (256
//    accumulators per lane), or BN = 128 with two workgroups per compute unit.
//
// Global -> LDS uses buffer loads with LDS destination (no VGPR staging). The range-checked part of each
// load's byte offset is its VGPR operand (the SGPR offset is outside the check): reads past this
// workgroup's row blocks and past the end of X return zeros without touching memory, so M/N tails need no
// branches in the main loop (columns past N only feed output columns that are never stored), and the loads
// the pipeline issues past the last tile are pushed out of range on purpose.
//   A (compressed values): the weight is stored as 1 KB tiles in the lane order of the smfmac A
//     operand (16 rows x 64 dense columns), so each tile is one contiguous 64-lane copy, and a
//     lane's ds_read_b128 of its operand is conflict-free.
//   metadata: 128 B tiles in lane order; a lane reads four fragments' 16-bit indices at once with
//     ds_read_b64_tr_b16 (16 lanes x 4 tiles transposed, so a lane gets its own index from each tile, two
//     to a register) and the smfmac's abid field selects the half.
//   B tile (X, 64 rows x 256 bf16 = 512 B per row; 128 bf16 = 256 B in the 128-wide tile): row-major
//     with the 32-byte units of row k stored at unit ^ v(k), v(k) = 2 (k & 3) + ((k >> 3) & 1) (< 8,
//     so a unit stays in its row for either width). One transposing read (below) takes 16 rows x 32
//     bytes, rows 8q + {0..3} for q = 0..3; v puts them in 8 distinct 32-byte bank groups (two rows
//     each, the minimum for 512 bytes). In global memory every 4 consecutive lanes of a load still
//     read one aligned 64-byte run (v only swaps its two halves or moves it whole).
// The B operand (lane = column, 16 k values in two halves of 8) comes from four ds_read_b64_tr_b16:
// in each 16-lane group, lane s points at row k0 + s/4, columns c0 + 4(s%4); the instruction hands
// lane i the four consecutive k of column c0 + i.
//
// Token-major X (N x K, the nn.Linear layout) needs no transposing read: the B tile is 256 token rows
// x 64 k (128 B per row), and a lane's operand is two 16-byte runs of its token's row (k = 8q .. +7
// and 32 + 8q .. +7), two ds_read_b128. Row n's 16-byte units sit at unit ^ f(n), f(n) = ((n >> 1) & 7)
// ^ 4 (n & 1): the 16 rows of one read group then use every 16-byte bank slot once per row parity (and
// 8 consecutive rows 8 distinct slots). The output Y (N x M) takes each accumulator's 4 consecutive
// rows of M as one 8- or 16-byte store, with no transposes. K must be a multiple of 64 there (inside a
// row the range check cannot stop at K).
//
// A batch of products sharing the weight (1x1 conv over B images) adds the batch to the tile index.
//
// Persistent: each workgroup (one or two per CU) walks its tiles (p, p + G, p + 2G, ... in a numbering where the
// workgroups of one XCD -- workgroup p runs on XCD p % 8 -- hold neighbouring tiles at the same time,
// walked in groups of 8 tile-rows, so A and B tiles are re-read from that XCD's L2). The three-stage
// LDS pipeline runs across tile boundaries: the last stages of a tile load the first stages of the
// next, and the epilogue works from registers only (4 x 4 transposes inside lane quads by DPP, then
// 8- or 16-byte stores), so its stores drain while the next tile computes.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace tiled_bf16 {

constexpr int BM = 256, BK = 64;
constexpr int WM = 128;
constexpr int FM = WM / 16;
constexpr int A_BYTES = BM * BK;          // BK/2 bf16 values per row = BK bytes
constexpr int META_BYTES = BM * BK / 8;   // 4 bits per group of 4
constexpr int GROUP_M = 8;

// Tile width BN (N columns of a workgroup tile): 256 (waves of 128 x 128), or 128 (waves of 128 x 64),
// which halves a tile's work for shapes whose 256-wide tiles leave most compute units idle in a last
// partial turn. The narrower stage (34 KB) leaves room for four LDS buffers.
// OCC_ = 2: two workgroups per compute unit (two waves per SIMD, at most 256 registers each), with
// two stage buffers each (2 x 2 x 34 KB of LDS), for the 128-wide tile only: one workgroup's smfmacs can
// run while the other waits at its barrier or for its loads.
// WAVES_ = 8: one workgroup of eight waves (two per SIMD, a 2 x 4 grid of 128 x BN/4 wave tiles) shares the
// 256-wide tile's loads, for two waves per SIMD without halving the tile.
template <int BN_, int OCC_ = 1, int WAVES_ = 4>
struct Cfg {
    static_assert(WAVES_ == 4 && (OCC_ == 1 || BN_ == 128), "supported configurations");
    static constexpr int WAVES = WAVES_;
    static constexpr int BN = BN_, WN = BN_ / (WAVES_ / 2), FN = WN / 16;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int B_ROW = BN * 2;  // feature-major B tile row: 512 or 256 bytes
    static constexpr int STAGE_BYTES = A_BYTES + META_BYTES + B_BYTES;
    static constexpr int NBUF = OCC_ == 2 ? 2 : (BN == 256 ? 3 : 4);  // 3 x 50 KB, 4 x 34 KB, 2 x 34 KB
    static constexpr int B_LOADS = BN / 32;          // per wave: 1 KB of the B tile per load
    static constexpr int LOADS_PER_STAGE = 4 + 2 + B_LOADS;  // per wave: A, metadata, B
    // How a wave issues a stage's loads once the barrier has freed its buffer (measured on MI355X):
    //  0: in one burst (two workgroups per CU: interleaving cost 3-4 %);
    //  2: LPRE of them interleaved with the first FN - 2 blocks of the next stage, in proportion to the
    //     smfmac slots there, the rest with the last two blocks (four waves of 256 accumulators, eight
    //     fragment blocks per stage: 7-8 % faster than the burst on 11008 x 4096 x 4096 feature-major).
    static constexpr int SPREAD = OCC_ == 2 ? 0 : 2;
    static constexpr int LPRE = SPREAD == 2 ? LOADS_PER_STAGE - (2 * LOADS_PER_STAGE + FN / 2) / FN : 0;
};
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
    int64_t sxb, syb;  // batch strides (elements)
    int tilesM, tilesN, batch;
    int y_vec;  // Y base and row pitch allow 8-byte (bf16) / 16-byte (fp32) stores, 4 rows < 2^31 bytes
};

// Where the loads of one tile come from: its corner and the buffer descriptors of its compressed
// row blocks. `valid` is false past the workgroup's last tile (its loads are then pushed out of range).
struct TileDesc {
    int64_t m0, n0;
    const uint16_t* x;  // X and Y of the tile's batch entry
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

// 16-byte unit swizzle of token row n of a token-major B tile (see the top of the file).
__device__ __forceinline__ int tm_swz(int n) { return ((n >> 1) & 7) ^ ((n & 1) << 2); }

// Per-lane parts of the load offsets (the uniform parts go into the SGPR offset operand).
struct LoadOffsets {
    uint32_t a;      // A tile: 16 * lane
    uint32_t m;      // metadata: 4 * (lane & 31) + (lane >> 5) * tiles * 128 (second tile of the pair)
    // feature-major, 256 wide: row pair (lane >> 5) * row pitch + 16 * swizzled chunk, by row & 3 >> 1 and
    // row >> 3 & 1; 128 wide (b[0], b[1]): row quad (lane >> 4) * row pitch + 16 * swizzled chunk, by
    // row >> 3 & 1; token-major (b[0], b[1]): (lane >> 3) * row pitch + 16 * swizzled unit, by row >> 3 & 1
    uint32_t b[4];
};

template <bool TM, int BNT>
__device__ __forceinline__ LoadOffsets load_offsets(const Args& a, int lane) {
    LoadOffsets o;
    const int tiles = (int)((a.K + BK - 1) / BK);
    o.a = 16 * lane;
    o.m = 4 * (lane & 31) + (lane >> 5) * tiles * 128;
    if constexpr (TM) {
        // lane i of a load lands in token row 8h + i / 8 of the tile, 16-byte slot i % 8, and reads the
        // unit that belongs there; only (row >> 3) & 1 = h & 1 changes the swizzle between loads
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int row = 8 * h + (lane >> 3);
            o.b[h] = (uint32_t)((lane >> 3) * a.ldx * 2 + 16 * ((lane & 7) ^ tm_swz(row)));
        }
        o.b[2] = o.b[3] = 0;
    } else if constexpr (BNT == 128) {
        // lane i of a load lands in row (i >> 4) of a quad of 256-byte rows, 16-byte slot i & 15; the
        // quads of one wave's loads differ in (row >> 3) & 1 only (row & 3 = i >> 4 in each)
        const int pc = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int row = (lane >> 4) + 8 * h;
            const int v = ((row & 3) << 1) | ((row >> 3) & 1);
            o.b[h] = (uint32_t)((lane >> 4) * a.ldx * 2 + 16 * (pc ^ (2 * v)));
        }
        o.b[2] = o.b[3] = 0;
    } else {
        const int pc = lane & 31;  // 16-byte slot in the LDS row
#pragma unroll
        for (int h = 0; h < 4; h++) {
            // a row with the same (row & 3) and (row >> 3) & 1 as this lane's row of the pair
            const int row = 2 * (h & 1) + (lane >> 5) + 8 * (h >> 1);
            const int v = ((row & 3) << 1) | ((row >> 3) & 1);
            const int lc = pc ^ (2 * v);  // 16-byte chunk of the X row
            o.b[h] = (uint32_t)((lane >> 5) * a.ldx * 2 + 16 * lc);
        }
    }
    return o;
}

// The loads of one stage (wave-uniform): the stage buffer, the three buffer descriptors and the stage's
// index. td.rA / td.rM cover the compressed tiles of the tile's row blocks (at most 16; tile (b, s) of
// block b at (b * tiles + s) * 1 KB of values and * 128 B of metadata). When td is not valid (past the
// workgroup's last tile) the offsets get bit 31 set, past every record count, so the loads return
// zeros without memory traffic (and X's record count is 0).
struct StageLoads {
    i32x4 rA, rM, rB;
    uint32_t lds, past;
    int s, tiles;
};

__device__ __forceinline__ StageLoads plan_stage(uint32_t lds, const Args& a, const TileDesc& td, int s) {
    StageLoads p;
    const int64_t k0 = (int64_t)s * BK;
    p.lds = lds;
    p.past = td.valid ? 0u : 0x80000000u;
    p.s = s;
    p.tiles = (int)((a.K + BK - 1) / BK);
    p.rA = td.rA;
    p.rM = td.rM;
    // X's exact extent from this stage's corner ((K - 1) rows of pitch ldx plus N elements); make_rsrc
    // rounds it up to whole dwords (the range check passes a dword only if all of it is in range)
    p.rB = make_rsrc(td.x + k0 * a.ldx + td.n0, td.valid ? ((a.K - 1 - k0) * a.ldx + a.N - td.n0) * 2 : 0);
    return p;
}

// Load number `ord` (0 .. LOADS_PER_STAGE - 1) of this wave's share of a stage: first the A tiles, then
// the metadata, then the B rows (feature-major X).
template <int BNT>
__device__ __forceinline__ void issue_load(const StageLoads& p, const Args& a, int ord, int wave, const LoadOffsets& lo) {
    constexpr int NA = 4, NM = 2;
    if (ord < NA) {
        // A: one 1 KB tile per 16-row block, copied as is (it is already in lane order)
        const int b = 4 * wave + ord;
        dma16(p.lds + b * 1024, lo.a + (((uint32_t)(b * p.tiles + p.s) * 1024u) | p.past), p.rA);
    } else if (ord < NA + NM) {
        // metadata: one 128 B tile per block; 4 blocks per wave, two per dword instruction
        const int b = 4 * wave + 2 * (ord - NA);
        dma4(p.lds + A_BYTES + b * 128, lo.m + (((uint32_t)(b * p.tiles + p.s) * 128u) | p.past), p.rM);
    } else if constexpr (BNT == 128) {
        // B: 64 rows x 256 B; rows 16 wave .. +15, four rows per load (rows 16 wave + 4h + lane / 16:
        // row & 3 = lane / 16, (row >> 3) & 1 = h >> 1)
        const int h = ord - NA - NM;
        const int row = 16 * wave + 4 * h;
        dma16(p.lds + A_BYTES + META_BYTES + row * 256, lo.b[h >> 1] + (uint32_t)(row * a.ldx * 2), p.rB);
    } else {
        // B: 64 rows x 512 B; rows 16 wave .. +15, two rows per load (rows 16 wave + 2h + lane / 32:
        // row & 3 = 2 (h & 1) + lane / 32, (row >> 3) & 1 = h >> 2)
        const int h = ord - NA - NM;
        const int row = 16 * wave + 2 * h;
        dma16(p.lds + A_BYTES + META_BYTES + row * 512, lo.b[(h & 1) | ((h >> 2) << 1)] + (uint32_t)(row * a.ldx * 2),
              p.rB);
    }
}

// Loads [O0, O1) of a stage, back to back.
template <int BNT, int O0, int O1>
__device__ __forceinline__ void issue_loads(const StageLoads& p, const Args& a, int wave, const LoadOffsets& lo) {
#pragma unroll
    for (int k = O0; k < O1; k++) issue_load<BNT>(p, a, k, wave, lo);
}

// Tile descriptor of logical tile L (-1: none). Batch entries follow each other; inside one, tiles
// are walked in groups of GROUP_M tile-rows, column by column inside a group.
template <bool OUT_FP32, int BNT>
__device__ __forceinline__ TileDesc tile_desc(const Args& a, int L) {
    TileDesc td;
    td.valid = L >= 0;
    const int per = a.tilesM * a.tilesN;
    const int bt = L >= 0 ? L / per : 0;
    const int Lc = L >= 0 ? L - bt * per : 0;
    td.x = a.X + bt * a.sxb;
    td.y = static_cast<char*>(a.Y) + bt * a.syb * (OUT_FP32 ? 4 : 2);
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
    td.rM = make_rsrc(a.meta + (td.m0 / 16) * tiles * 128, blocks * tiles * 128);
    return td;
}

// Lane-dependent LDS byte offsets used by compute_stage (computed once per kernel).
template <int FNT, int BROW>  // fragments per wave, bytes per row of the feature-major B tile
struct LaneOffsets {
    int a;        // A fragment of block wm0/16: block * 1024 + lane * 16
    int m;        // metadata: the transposing read of blocks wm0/16 .. +3, A_BYTES + (wm0 / 16) * 128 +
                  // 128 ((lane & 15) >> 2) + 32 (lane >> 4) + 8 (lane & 3) (+512: the next four blocks)
    int b[FNT];   // B fragment j, first read (t = 0): row part + swizzled column part; token-major: the
                  // two reads of fragment 0 (b[0], b[1]; fragment j adds 16 rows x 128 B)
};

template <bool TM, int FNT, int BROW>
__device__ __forceinline__ LaneOffsets<FNT, BROW> lane_offsets(int wm0, int wn0, int lane) {
    const int r = lane & 15, q = lane >> 4;
    LaneOffsets<FNT, BROW> o;
    o.a = (wm0 >> 4) * 1024 + lane * 16;
    o.m = A_BYTES + (wm0 >> 4) * 128 + 128 * (r >> 2) + 32 * q + 8 * (r & 3);
    if constexpr (TM) {
        const int base = A_BYTES + META_BYTES + (wn0 + r) * 128, u = q ^ tm_swz(r);
        o.b[0] = base + 16 * u;
        o.b[1] = base + 16 * (u ^ 4);
#pragma unroll
        for (int j = 2; j < FNT; j++) o.b[j] = 0;
        return o;
    }
    // read t of group q covers rows 8q + 4(t&1) + 32(t>>1) + r/4, which all have the row & 3 and
    // (row >> 3) & 1 of row0, so the unit swizzle is fixed per lane and t only adds immediates
    constexpr int B_ROW = BROW;
    const int row0 = 8 * q + (r >> 2);
    const int v = ((row0 & 3) << 1) | ((row0 >> 3) & 1);
#pragma unroll
    for (int j = 0; j < FNT; j++) {
        const int col = wn0 + 16 * j + 4 * (r & 3);  // first of the 4 columns this lane points at
        o.b[j] = A_BYTES + META_BYTES + row0 * B_ROW + (((col >> 4) ^ v) << 5) + 2 * (col & 15);
    }
    return o;
}

// Operands of one stage held in registers: the 8 A fragments and their indices, packed two to a register
// (fragment i in half i & 1 of idx[i / 2]).
struct AFrags {
    bf16x8 a[FM];
    uint32_t idx[FM / 2];
};

typedef __attribute__((address_space(3))) char lds_char;

// Indices of fragments 4q .. 4q + 3 from the transposing read at p: element k of the 16-lane transpose is the
// lane's 16-bit index in tile 4q + k, so the two registers hold fragments (4q, 4q + 1) and (4q + 2, 4q + 3).
__device__ __forceinline__ u32x2 read_idx4(const lds_char* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// smfmac of fragment i (unrolled, so the branch folds) with its index from the packed registers.
__device__ __forceinline__ f32x4 smfmac_p(const AFrags& f, int i, const bf16x16& b, const f32x4& c) {
    return (i & 1) ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(f.a[i], b, c, (int)f.idx[i >> 1], 0, 1)
                   : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(f.a[i], b, c, (int)f.idx[i >> 1], 0, 0);
}

// A lane's LDS address for this stage's buffer, made opaque to the optimizer: otherwise it hoists
// the (lane offset + immediate) sums of every read out of the K loop, 32 loop-invariant registers
// for B alone, instead of folding the immediates into the reads' offset fields.
__device__ __forceinline__ uint32_t stage_addr(uint32_t buf, int off) {
    uint32_t v = buf + (uint32_t)off;
    asm volatile("" : "+v"(v));
    return v;
}

template <int FNT, int BROW>
__device__ __forceinline__ void read_a(uint32_t buf, const LaneOffsets<FNT, BROW>& o, AFrags& f) {
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(buf, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(buf, o.m);
#pragma unroll
    for (int i = 0; i < FM; i++)
        f.a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
    const u32x2 m0 = read_idx4(pm), m1 = read_idx4(pm + 512);
    f.idx[0] = m0[0];
    f.idx[1] = m0[1];
    f.idx[2] = m1[0];
    f.idx[3] = m1[1];
}

// B fragment j (16 columns x 64 k) of the stage in buffer `buf`: four transposing reads, or, token-
// major, two 16-byte reads of the lane's token row.
template <bool TM, int FNT, int BROW>
__device__ __forceinline__ bf16x16 read_b(uint32_t buf, const LaneOffsets<FNT, BROW>& o, int j) {
    if constexpr (TM) {
        typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
        const lds_char* p0 = (const lds_char*)(size_t)stage_addr(buf, o.b[0]);
        const lds_char* p1 = (const lds_char*)(size_t)stage_addr(buf, o.b[1]);
        const u32x4 lo = *reinterpret_cast<lds_u32x4*>(p0 + j * 2048);
        const u32x4 hi = *reinterpret_cast<lds_u32x4*>(p1 + j * 2048);
        return __builtin_bit_cast(bf16x16, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
    constexpr int B_ROW = BROW;
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

// Loads still to be issued for an earlier stage: this wave issues a stage's loads partly after the barrier
// that frees its buffer and partly during the first fragment blocks of the next stage (see `stage`).
// nxt: the loads belong to the tile after the current one; s: their stage index in that tile.
struct Pending {
    bool nxt;
    int s;
};

// Fragment block j (FM smfmacs), with loads O0 + k, k < N, of `p` interleaved: a region of R smfmac slots
// starting at slot `first` of this block takes load k after its slot (k * R) / N, so the wave never
// queues more than a load or two at the texture unit while it has smfmacs to issue.
template <int BNT, int FNT, int N, int R, int O0>
__device__ __forceinline__ void mfma_block(f32x4 (&acc)[FM][FNT], const AFrags& f, const bf16x16& b, int j, int first,
                                           const StageLoads& p, const Args& a, int wave, const LoadOffsets& lo) {
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][j] = smfmac_p(f, i, b, acc[i][j]);
#pragma unroll
        for (int k = 0; k < N; k++)
            if ((k * R) / N == first + i) issue_load<BNT>(p, a, O0 + k, wave, lo);
        if constexpr (N > 0) __builtin_amdgcn_sched_barrier(0);
    }
}

// One K stage of the feature-major loop: stage s of the current tile, g-th stage of the workgroup overall
// (selects the buffer).
// The loads of stage s + NBUF of the current tile (or, past its end, stage s + NBUF - S of the next) go
// into this stage's buffer once the barrier has freed it, in one of the patterns Cfg::SPREAD selects;
// in pattern 2 the last LPRE of them are issued during the first F - 2 blocks of the next stage (the
// `pend` loads; three buffers). The vmcnt wait is the same in every pattern: at the barrier of stage g
// the newest LOADS_PER_STAGE loads are exactly those of stage g + NBUF - 1. No branches.
template <int BNT, int OCC>
__device__ __forceinline__ void stage(uint32_t l0, const Args& a, const TileDesc& cur_t, const TileDesc& next_t, int s,
                                      int S, int g, f32x4 (&acc)[FM][Cfg<BNT, OCC>::FN], AFrags& f, bf16x16 (&rb)[4],
                                      const LaneOffsets<Cfg<BNT, OCC>::FN, Cfg<BNT>::B_ROW>& o, int wave,
                                      const LoadOffsets& lo, Pending& pend) {
    using C = Cfg<BNT, OCC>;
    constexpr int F = C::FN, NB = C::NBUF, L = C::LOADS_PER_STAGE;
    constexpr int LPRE = C::LPRE, LPOST = L - LPRE;
    const int cb = g % NB;
    const uint32_t cur = l0 + cb * C::STAGE_BYTES;
    const uint32_t nxt = l0 + (cb == NB - 1 ? 0 : cb + 1) * C::STAGE_BYTES;
    StageLoads pp;
    if constexpr (LPRE > 0)
        pp = plan_stage(l0 + (cb == 0 ? NB - 1 : cb - 1) * C::STAGE_BYTES, a, pend.nxt ? next_t : cur_t, pend.s);
#pragma unroll
    for (int j = 0; j < F - 2; j++) {
        rb[(j + 2) & 3] = read_b<false>(cur, o, j + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block<BNT, F, LPRE, (F - 2) * FM, LPOST>(acc, f, rb[j & 3], j, j * FM, pp, a, wave, lo);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's reads of stage g are done
    wait_vmcnt<(NB - 2) * L>();                   // stage g+1 has landed (later ones may be in flight)
    __builtin_amdgcn_s_barrier();
    const bool here = s + NB < S;
    pend.nxt = !here;
    pend.s = here ? s + NB : s + NB - S;
    const StageLoads np = plan_stage(cur, a, here ? cur_t : next_t, pend.s);
    if constexpr (C::SPREAD == 0) issue_loads<BNT, 0, L>(np, a, wave, lo);
    constexpr int LI = C::SPREAD == 0 ? 0 : LPOST;  // loads interleaved with the last two blocks
    rb[0] = read_b<false>(nxt, o, 0);
    rb[1] = read_b<false>(nxt, o, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block<BNT, F, LI, 2 * FM, 0>(acc, f, rb[(F - 2) & 3], F - 2, 0, np, a, wave, lo);
    __builtin_amdgcn_sched_barrier(0);
    // last block: once fragment i has been used for the last time, reload it (and its index) from the
    // next stage, so one A register set serves the whole pipeline
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(nxt, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(nxt, o.m);
    u32x2 m0, m1;  // the next stage's indices of fragments 0-3 and 4-7, read once this block has used the old ones
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][F - 1] = smfmac_p(f, i, rb[(F - 1) & 3], acc[i][F - 1]);
        f.a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
        if (i == 3) m0 = read_idx4(pm);
        if (i == FM - 1) m1 = read_idx4(pm + 512);
#pragma unroll
        for (int k = 0; k < LI; k++)
            if ((k * 2 * FM) / LI == FM + i) issue_load<BNT>(np, a, k, wave, lo);
        __builtin_amdgcn_sched_barrier(0);
    }
    f.idx[0] = m0[0];
    f.idx[1] = m0[1];
    f.idx[2] = m1[0];
    f.idx[3] = m1[1];
}

// ---------------------------------------------------------------- epilogue
// From registers, four fragments (64 columns) at a time. The store path issues one request per lane
// quad when the quad's 4 lanes fall in one 128-byte line and one per lane otherwise (measured: a
// store instruction whose 64 lanes touch 16 rows costs about 3x one that touches 4), so each lane quad
// is given one output row: the quad transposes of each fragment leave lane (q, 4a + b) with row 4q + b,
// columns 4a .. 4a+3 of fragment f in slot f, and a quad transpose across the slots then gives lane
// (q, 4a + x) row 4q + s, columns 16x + 4a .. +3 in slot s. A store of slot s thus writes 4 rows x 64
// columns, whole 128-byte lines (a line is never cached half written, which with power-of-two row
// pitches led to lines evicted and written back twice), one line per quad for bf16 and two for fp32.
// No LDS is used, so the next tile's loads can land in the stage buffers meanwhile.
// FULL: the wave's whole 128 x 128 block lies inside Y and vector stores are allowed (then the row
// offsets of a lane quad fit 32 bits); otherwise every element is bounds-checked. The vector stores carry
// the non-temporal hint: Y is not read again by this kernel, and streaming its lines out instead of
// leaving them dirty in L2 shortens the drain after the last tiles (measured: 3072 x 768 x 6304
// token-major 33.7 -> 32.2 us, 4096^3 87.6 -> 82.5 us).
template <bool OUT_FP32, bool FULL, int FNT>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[FM][FNT], const Args& a, char* y, int64_t mw, int64_t nw,
                                           int lane) {
    constexpr int W = OUT_FP32 ? 4 : 2, ES = OUT_FP32 ? 4 : 2;
    const int q = lane >> 4, r = lane & 15, b = r & 3, a4 = r >> 2;
    const uint32_t sel = half_sel(b);
    char* const y0 = y + (mw * a.ldy + nw) * ES;  // wave-uniform corner
    // lane (q, 4 a4 + b) stores row 4q + s, columns 16 b + 4 a4 .. +3 of the 64-column group
    const uint32_t lane_off = FULL ? (uint32_t)((4 * q * a.ldy + 16 * b + 4 * a4) * ES) : 0u;
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int jg = 0; jg < FNT / 4; jg++) {
            uint32_t v[4][W];
#pragma unroll
            for (int f = 0; f < 4; f++) {
                const f32x4 c = acc[i][4 * jg + f];
                if constexpr (OUT_FP32) {
#pragma unroll
                    for (int t = 0; t < 4; t++) v[f][t] = __float_as_uint(c[t]);
                    quad_transpose(v[f], b);
                } else {
                    const float e[4] = {c[0], c[1], c[2], c[3]};
                    quad_transpose_bf16(e, v[f], b, sel);
                }
            }
            slot_transpose4<W>(v, b);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                if constexpr (FULL) {
                    char* const p = y0 + ((16 * i + s) * a.ldy + 64 * jg) * ES + lane_off;
                    if constexpr (OUT_FP32)
                        __builtin_nontemporal_store(u32x4{v[s][0], v[s][1], v[s][2], v[s][3]}, reinterpret_cast<u32x4*>(p));
                    else
                        __builtin_nontemporal_store(u32x2{v[s][0], v[s][1]}, reinterpret_cast<u32x2*>(p));
                } else {
                    const int64_t m = mw + 16 * i + 4 * q + s, n = nw + 64 * jg + 16 * b + 4 * a4;
                    if (m < a.M) {
#pragma unroll
                        for (int k = 0; k < 4; k++) {
                            if (n + k >= a.N) continue;
                            const uint32_t w = v[s][OUT_FP32 ? k : k >> 1];
                            if constexpr (OUT_FP32)
                                reinterpret_cast<uint32_t*>(y)[m * a.ldy + n + k] = w;
                            else
                                reinterpret_cast<uint16_t*>(y)[m * a.ldy + n + k] = (uint16_t)(k & 1 ? w >> 16 : w);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one row block of fragments at a time (bounded live registers)
    }
}

// Token-major epilogue: Y is N x M, and each accumulator (column n, rows 4q .. 4q+3 of M) is 4
// consecutive elements of token row n. The lanes of a quad hold 4 different rows n, so a quad
// transpose across four row fragments (slots i) gives lane (q, 4c + x) token row 4c + s, elements
// 16x + 4q .. +3 of the 64 M-columns of the fragment group in slot s: each quad's stores then fall in
// one 128-byte line (bf16) or two (fp32), and each store instruction covers 16 token rows x 64
// elements, whole lines.
template <bool OUT_FP32, bool FULL, int FNT>
__device__ __forceinline__ void store_tile_tm(const f32x4 (&acc)[FM][FNT], const Args& a, char* y, int64_t mw,
                                              int64_t nw, int lane) {
    constexpr int ES = OUT_FP32 ? 4 : 2, W = OUT_FP32 ? 4 : 2;
    const int q = lane >> 4, r = lane & 15, x = r & 3, c = r >> 2;
    char* const y0 = y + (nw * a.ldy + mw) * ES;  // wave-uniform corner
    const uint32_t lane_off = FULL ? (uint32_t)((4 * c * a.ldy + 16 * x + 4 * q) * ES) : 0u;
#pragma unroll
    for (int j = 0; j < FNT; j++) {
#pragma unroll
        for (int ig = 0; ig < FM / 4; ig++) {
            uint32_t v[4][W];
#pragma unroll
            for (int f = 0; f < 4; f++) {
                const f32x4 e = acc[4 * ig + f][j];
                if constexpr (OUT_FP32) {
#pragma unroll
                    for (int t = 0; t < 4; t++) v[f][t] = __float_as_uint(e[t]);
                } else {
                    v[f][0] = pack_bf16x2_rne(e[0], e[1]);
                    v[f][1] = pack_bf16x2_rne(e[2], e[3]);
                }
            }
            slot_transpose4<W>(v, x);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                if constexpr (FULL) {
                    char* const p = y0 + ((16 * j + s) * a.ldy + 64 * ig) * ES + lane_off;
                    if constexpr (OUT_FP32)
                        __builtin_nontemporal_store(u32x4{v[s][0], v[s][1], v[s][2], v[s][3]}, reinterpret_cast<u32x4*>(p));
                    else
                        __builtin_nontemporal_store(u32x2{v[s][0], v[s][1]}, reinterpret_cast<u32x2*>(p));
                } else {
                    const int64_t n = nw + 16 * j + 4 * c + s, m = mw + 64 * ig + 16 * x + 4 * q;
                    if (n < a.N) {
#pragma unroll
                        for (int t = 0; t < 4; t++) {
                            if (m + t >= a.M) continue;
                            const uint32_t w = v[s][OUT_FP32 ? t : t >> 1];
                            if constexpr (OUT_FP32)
                                reinterpret_cast<uint32_t*>(y)[n * a.ldy + m + t] = w;
                            else
                                reinterpret_cast<uint16_t*>(y)[n * a.ldy + m + t] = (uint16_t)(t & 1 ? w >> 16 : w);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The feature-major loop (X K x N): 256 x 256 tiles with four waves of 128 x 128, or 256 x 128 tiles with two
// workgroups per compute unit.
template <bool OUT_FP32, int BNT, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gemm_bf16_tiled_kernel(Args a) {
    using C = Cfg<BNT, OCC>;
    constexpr int NB = C::NBUF, F = C::FN;
    __shared__ __attribute__((aligned(16))) char smem[NB * C::STAGE_BYTES];
    // LDS byte address of the first stage buffer (for the LDS-destination loads)
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;

    const int p = blockIdx.x;
    int L = tile_of(a, p, 0);
    if (L < 0) return;  // whole workgroup
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm0 = (wave / 2) * WM, wn0 = (wave % 2) * C::WN;
    const LaneOffsets<F, C::B_ROW> o = lane_offsets<false, F, C::B_ROW>(wm0, wn0, lane);
    const LoadOffsets lo = load_offsets<false, BNT>(a, lane);
    const int S = (int)((a.K + BK - 1) / BK);

    f32x4 acc[FM][F];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < F; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over K stages of 64 columns, NB LDS buffers (2 with two workgroups per CU, else
    // 3 for 256-wide tiles and 4 for 128-wide; the workgroup's g-th stage in buffer g % NB), continued
    // across the workgroup's tiles:
    //  - the loads of stage g+NB go out once every wave has finished reading stage g, i.e. at the
    //    barrier placed before the last two fragment blocks of stage g, so each stage's loads have
    //    about NB - 1 stages of compute to land;
    //  - that barrier also publishes stage g+1 (each wave first waits for its own loads of it), so
    //    stage g+1's A fragments, indices and first B fragments are read while the last 16 smfmacs of
    //    stage g run;
    //  - inside a stage, B fragment j+2 is read while fragment j is multiplied (ring of 4).
    // With fewer than NB stages per tile every workgroup has one tile (see the launcher), so the
    // prologue's loads past the tile's stages (next_t invalid) only zero-fill.
    TileDesc cur_t = tile_desc<OUT_FP32, BNT>(a, L);
    TileDesc next_t = tile_desc<OUT_FP32, BNT>(a, tile_of(a, p, 1));
#pragma unroll
    for (int i = 0; i < NB - 1; i++)
        issue_loads<BNT, 0, C::LOADS_PER_STAGE>(
            plan_stage(l0 + i * C::STAGE_BYTES, a, S > i ? cur_t : next_t, S > i ? i : 0), a, wave, lo);
    wait_vmcnt<(NB - 2) * C::LOADS_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    // stage NB - 1: the loads a stage issues after its barrier; the first stage issues the rest
    Pending pend{S <= NB - 1, S > NB - 1 ? NB - 1 : 0};
    issue_loads<BNT, 0, C::LOADS_PER_STAGE - C::LPRE>(
        plan_stage(l0 + (NB - 1) * C::STAGE_BYTES, a, pend.nxt ? next_t : cur_t, pend.s), a, wave, lo);

    AFrags fa;
    bf16x16 rb[4];
    read_a(l0, o, fa);
    rb[0] = read_b<false>(l0, o, 0);
    rb[1] = read_b<false>(l0, o, 1);
    int g = 0;
    for (int k = 1;; k++) {
        for (int s = 0; s < S; s++, g++)
            stage<BNT, OCC>(l0, a, cur_t, next_t, s, S, g, acc, fa, rb, o, wave, lo, pend);
        // epilogue from registers; the next tile's first stages are in flight meanwhile
        {
            const int64_t mw = cur_t.m0 + wm0, nw = cur_t.n0 + wn0;
            if ((mw + WM <= a.M) && (nw + C::WN <= a.N) && a.y_vec)
                store_tile<OUT_FP32, true>(acc, a, cur_t.y, mw, nw, lane);
            else
                store_tile<OUT_FP32, false>(acc, a, cur_t.y, mw, nw, lane);
        }
        if (!next_t.valid) break;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < F; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        cur_t = next_t;
        pend.nxt = false;  // the pending loads' tile (the next one) is now the current one
        next_t = tile_desc<OUT_FP32, BNT>(a, tile_of(a, p, k + 1));
    }
    wait_vmcnt<0>();  // the zero-filling loads past the last tile have landed before the workgroup ends
}

// ---------------------------------------------------------------- token-major main loop
// Token-major X (N x K) with waves of 128 x 64 (two per SIMD): 256-wide tiles with eight waves and three stage
// buffers, or 128-wide tiles with four waves, two stage buffers and two workgroups per compute unit. Per-stage
// scalar work is kept to the stage's soffsets and buffer rotation: the buffer descriptors are made once per tile
// (record count 0 for a tile past the last one), the lane-dependent part of every load offset (the part the range
// check covers: the row block of A and metadata, the token row of X) is fixed per kernel, and the stage's advance
// along K (s * 1 KB of A tiles, s * 128 B of metadata and of each X row) goes into the SGPR offset operand.
__device__ __forceinline__ void dma16s(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}
__device__ __forceinline__ void dma4s(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

template <int BN>
struct TmCfg {
    static constexpr int WAVES = BN / 32;  // 8 or 4: two waves per SIMD either way (one or two workgroups per CU)
    static constexpr int WN = 64, FN = 4;
    static constexpr int STAGE_BYTES = A_BYTES + META_BYTES + BK * BN * 2;
    static constexpr int NBUF = BN == 256 ? 3 : 2;
    static constexpr int NA = 16 / WAVES, NM = 8 / WAVES, NBL = BN / 8 / WAVES;  // loads per wave per stage
    static constexpr int L = NA + NM + NBL;
};

struct TmTile {
    int64_t m0, n0;
    char* y;
    i32x4 rA, rM, rB;
    bool valid;
};

template <bool OUT_FP32, int BNT>
__device__ __forceinline__ TmTile tm_tile(const Args& a, int L) {
    const TileDesc d = tile_desc<OUT_FP32, BNT>(a, L);
    TmTile t;
    t.m0 = d.m0;
    t.n0 = d.n0;
    t.y = d.y;
    t.valid = d.valid;
    t.rA = d.rA;
    t.rM = d.rM;
    t.rB = make_rsrc(d.x + d.n0 * a.ldx, ((a.N - 1 - d.n0) * a.ldx + a.K) * 2);
    if (!d.valid) {
        t.rA[2] = 0;
        t.rM[2] = 0;
        t.rB[2] = 0;
    }
    return t;
}

// Load k (compile-time) of this wave's share of one stage into the buffer at byte offset buf.
template <int BN, int k>
__device__ __forceinline__ void tm_load(uint32_t buf, const TmTile& t, uint32_t soffA, uint32_t soffMB, int wave,
                                        uint32_t tiles, uint32_t ldx2, const LoadOffsets& lo) {
    using C = TmCfg<BN>;
    if constexpr (k < C::NA) {
        const uint32_t b = C::NA * wave + k;
        dma16s(buf + b * 1024, lo.a + b * tiles * 1024u, t.rA, soffA);
    } else if constexpr (k < C::NA + C::NM) {
        const uint32_t b = 2 * (C::NM * wave + (k - C::NA));
        dma4s(buf + A_BYTES + b * 128, lo.m + b * tiles * 128u, t.rM, soffMB);
    } else {
        constexpr int h = k - C::NA - C::NM;
        const uint32_t r0 = 8 * (C::NBL * wave + h);
        dma16s(buf + A_BYTES + META_BYTES + r0 * 128, lo.b[h & 1] + r0 * ldx2, t.rB, soffMB);
    }
}

template <int BN, int k0, int k1>
__device__ __forceinline__ void tm_loads(uint32_t buf, const TmTile& t, uint32_t soffA, uint32_t soffMB, int wave,
                                         uint32_t tiles, uint32_t ldx2, const LoadOffsets& lo) {
    if constexpr (k0 < k1) {
        tm_load<BN, k0>(buf, t, soffA, soffMB, wave, tiles, ldx2, lo);
        tm_loads<BN, k0 + 1, k1>(buf, t, soffA, soffMB, wave, tiles, ldx2, lo);
    }
}

// Loads interleaved with smfmac slot `slot` (0 .. 3 FM - 1) of the last three fragment blocks: load k after slot
// (k * 3 FM) / L.
template <int BN, int k>
__device__ __forceinline__ void tm_loads_at(int slot, uint32_t buf, const TmTile& t, uint32_t soffA, uint32_t soffMB,
                                            int wave, uint32_t tiles, uint32_t ldx2, const LoadOffsets& lo) {
    if constexpr (k < TmCfg<BN>::L) {
        if ((k * 3 * FM) / TmCfg<BN>::L == slot) tm_load<BN, k>(buf, t, soffA, soffMB, wave, tiles, ldx2, lo);
        tm_loads_at<BN, k + 1>(slot, buf, t, soffA, soffMB, wave, tiles, ldx2, lo);
    }
}

// One K stage: the current buffer `cur` (this stage), `nxt` (the next stage, published by this stage's barrier).
// The barrier sits after the first fragment block: B fragments 2 and 3 are read before it, so the rest of the
// stage's operand traffic (the next stage's B fragments 0 and 1, A fragments and indices, and this wave's
// loads of stage `ls` of tile `lt` into `cur`) spreads over the last three blocks.
template <int BN>
__device__ __forceinline__ void tm_stage(uint32_t l0, uint32_t cur, uint32_t nxt, const TmTile& lt, uint32_t ls,
                                         f32x4 (&acc)[FM][4], AFrags& f, bf16x16 (&rb)[4],
                                         const LaneOffsets<4, 256>& o, int wave, uint32_t tiles, uint32_t ldx2,
                                         const LoadOffsets& lo) {
    using C = TmCfg<BN>;
    constexpr int NB = C::NBUF, L = C::L;
    const uint32_t cb = l0 + cur, nb = l0 + nxt;
    rb[2] = read_b<true>(cb, o, 2);
    rb[3] = read_b<true>(cb, o, 3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++)
        acc[i][0] = smfmac_p(f, i, rb[0], acc[i][0]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the stage are done
    wait_vmcnt<(NB - 2) * L>();          // the next stage has landed
    __builtin_amdgcn_s_barrier();
    const uint32_t soffA = ls * 1024u, soffMB = ls * 128u;
    rb[0] = read_b<true>(nb, o, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][1] = smfmac_p(f, i, rb[1], acc[i][1]);
        tm_loads_at<BN, 0>(i, cb, lt, soffA, soffMB, wave, tiles, ldx2, lo);
        __builtin_amdgcn_sched_barrier(0);
    }
    rb[1] = read_b<true>(nb, o, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][2] = smfmac_p(f, i, rb[2], acc[i][2]);
        tm_loads_at<BN, 0>(FM + i, cb, lt, soffA, soffMB, wave, tiles, ldx2, lo);
        __builtin_amdgcn_sched_barrier(0);
    }
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(nb, o.a);
    const lds_char* pm = (const lds_char*)(size_t)stage_addr(nb, o.m);
    u32x2 m0, m1;  // the next stage's indices of fragments 0-3 and 4-7, read once this block has used the old ones
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][3] = smfmac_p(f, i, rb[3], acc[i][3]);
        f.a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
        if (i == 3) m0 = read_idx4(pm);
        if (i == FM - 1) m1 = read_idx4(pm + 512);
        tm_loads_at<BN, 0>(2 * FM + i, cb, lt, soffA, soffMB, wave, tiles, ldx2, lo);
        __builtin_amdgcn_sched_barrier(0);
    }
    f.idx[0] = m0[0];
    f.idx[1] = m0[1];
    f.idx[2] = m1[0];
    f.idx[3] = m1[1];
}

template <bool OUT_FP32, int BN>
__global__ __launch_bounds__(64 * TmCfg<BN>::WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16_tm_kernel(
    Args a) {
    using C = TmCfg<BN>;
    constexpr int NB = C::NBUF, W = C::WAVES, L = C::L, SB = C::STAGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[NB * SB];
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    const int p = blockIdx.x;
    int Lt = tile_of(a, p, 0);
    if (Lt < 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm0 = (wave / (W / 2)) * WM, wn0 = (wave % (W / 2)) * C::WN;
    const LaneOffsets<4, 256> o = lane_offsets<true, 4, 256>(wm0, wn0, lane);
    const LoadOffsets lo = load_offsets<true, BN>(a, lane);
    const int S = (int)(a.K / BK);
    const uint32_t tiles = (uint32_t)S, ldx2 = (uint32_t)(a.ldx * 2);

    f32x4 acc[FM][4];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    TmTile cur_t = tm_tile<OUT_FP32, BN>(a, Lt);
    TmTile nxt_t = tm_tile<OUT_FP32, BN>(a, tile_of(a, p, 1));
    // prologue: stages 0 .. NB - 1 (past the tile's stages: the next tile's first ones)
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const bool here = i < S;
        const uint32_t ls = here ? i : i - S;
        if (i == NB - 1) {
            wait_vmcnt<(NB - 2) * L>();
            __builtin_amdgcn_s_barrier();
        }
        tm_loads<BN, 0, L>(i * SB, here ? cur_t : nxt_t, ls * 1024u, ls * 128u, wave, tiles, ldx2, lo);
    }
    AFrags fa;
    bf16x16 rb[4];
    read_a(l0, o, fa);
    rb[0] = read_b<true>(l0, o, 0);
    rb[1] = read_b<true>(l0, o, 1);
    uint32_t cur = 0;
    for (int k = 1;; k++) {
        int s = 0;
        // stages whose barrier-time loads are this tile's stage s + NB
        for (; s < S - NB; s++) {
            const uint32_t nxt = cur == (NB - 1) * SB ? 0u : cur + SB;
            tm_stage<BN>(l0, cur, nxt, cur_t, (uint32_t)(s + NB), acc, fa, rb, o, wave, tiles, ldx2, lo);
            cur = nxt;
        }
        // the last NB stages load the next tile's first stages
        for (; s < S; s++) {
            const uint32_t nxt = cur == (NB - 1) * SB ? 0u : cur + SB;
            tm_stage<BN>(l0, cur, nxt, nxt_t, (uint32_t)(s + NB - S), acc, fa, rb, o, wave, tiles, ldx2, lo);
            cur = nxt;
        }
        {
            const int64_t mw = cur_t.m0 + wm0, nw = cur_t.n0 + wn0;
            if ((mw + WM <= a.M) && (nw + C::WN <= a.N) && a.y_vec)
                store_tile_tm<OUT_FP32, true>(acc, a, cur_t.y, mw, nw, lane);
            else
                store_tile_tm<OUT_FP32, false>(acc, a, cur_t.y, mw, nw, lane);
        }
        if (!nxt_t.valid) break;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        cur_t = nxt_t;
        nxt_t = tm_tile<OUT_FP32, BN>(a, tile_of(a, p, k + 1));
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------- dense reference (measurement only)
// A dense bf16 GEMM on v_mfma_f32_16x16x32_bf16 with the token-major sparse loop's tiling -- 256 x 256 workgroup
// tiles in the same persistent XCD-aware walk, eight waves of 128 x 64, 32 MFMAs per wave per stage, the barrier
// after the first fragment block, the same loads with an SGPR stage offset and the same epilogue -- so that its
// time against the sparse kernel's isolates what 2:4 sparsity changes (a 16 x 16 x 64 block is one smfmac
// instead of two MFMAs). K advances 32 per stage (one MFMA's depth) through four 32 KB stage buffers, about the
// bytes in flight of the sparse loop's three 50 KB ones. The weight is a dense copy in MFMA operand order: tiles
// of 16 rows x 32 columns (1 KB), byte range [16 l, 16 l + 16) = lane l's A operand (row l % 16, columns
// 8 (l / 16) .. +7), stored row block by row block and along K inside a block.
namespace dense_ref {
constexpr int BKD = 32, NB = 4, WAVES = 8, BN = 256;
constexpr int A_TILE = BM * BKD * 2;             // 16 KB
constexpr int STAGE_BYTES = A_TILE + BN * BKD * 2;  // + 256 token rows x 64 B
constexpr int NA = 2, NBL = 2, L = NA + NBL;     // loads per wave per stage (1 KB each)

// The B tile holds 64 B per token row; the 16-byte unit u of row n sits at u ^ ((n >> 2) & 3), so the 16 rows
// of one read group (one unit each) start in 16 distinct 4-bank groups.
struct Tile {
    int64_t m0, n0;
    char* y;
    i32x4 rA, rB;
    bool valid;
};

template <bool OUT_FP32>
__device__ __forceinline__ Tile tile(const Args& a, int L) {
    const TileDesc d = tile_desc<OUT_FP32, BN>(a, L);
    Tile t;
    t.m0 = d.m0;
    t.n0 = d.n0;
    t.y = d.y;
    t.valid = d.valid;
    const int64_t kt = a.K / BKD, blocks_left = (a.M + 15) / 16 - d.m0 / 16;
    const int64_t blocks = blocks_left < BM / 16 ? blocks_left : BM / 16;
    t.rA = make_rsrc(reinterpret_cast<const char*>(a.vals) + (d.m0 / 16) * kt * 1024, d.valid ? blocks * kt * 1024 : 0);
    t.rB = make_rsrc(d.x + d.n0 * a.ldx, d.valid ? ((a.N - 1 - d.n0) * a.ldx + a.K) * 2 : 0);
    return t;
}

template <int k>
__device__ __forceinline__ void load(uint32_t buf, const Tile& t, uint32_t soffA, uint32_t soffB, int wave, uint32_t kt,
                                     uint32_t ldx2, uint32_t la, uint32_t lb) {
    if constexpr (k < NA) {
        const uint32_t b = NA * wave + k;
        dma16s(buf + b * 1024, la + b * kt * 1024u, t.rA, soffA);
    } else {
        const uint32_t r0 = 16 * (NBL * wave + (k - NA));
        dma16s(buf + A_TILE + r0 * 64, lb + r0 * ldx2, t.rB, soffB);
    }
}

template <int k>
__device__ __forceinline__ void loads_at(int slot, uint32_t buf, const Tile& t, uint32_t soffA, uint32_t soffB, int wave,
                                         uint32_t kt, uint32_t ldx2, uint32_t la, uint32_t lb) {
    if constexpr (k < L) {
        if ((k * 3 * FM) / L == slot) load<k>(buf, t, soffA, soffB, wave, kt, ldx2, la, lb);
        loads_at<k + 1>(slot, buf, t, soffA, soffB, wave, kt, ldx2, la, lb);
    }
}

__device__ __forceinline__ bf16x8 read16(uint32_t addr) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                                          (const lds_char*)(size_t)stage_addr(addr, 0)));
}

__device__ __forceinline__ void stage(uint32_t l0, uint32_t cur, uint32_t nxt, const Tile& lt, uint32_t ls,
                                      f32x4 (&acc)[FM][4], bf16x8 (&fa)[FM], bf16x8 (&rb)[4], uint32_t oa, uint32_t ob,
                                      int wave, uint32_t kt, uint32_t ldx2, uint32_t la, uint32_t lb) {
    const uint32_t cb = l0 + cur, nb = l0 + nxt;
    rb[2] = read16(cb + ob + 2 * 1024);
    rb[3] = read16(cb + ob + 3 * 1024);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++) acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], rb[0], acc[i][0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    wait_vmcnt<(NB - 2) * L>();
    __builtin_amdgcn_s_barrier();
    const uint32_t soffA = ls * 1024u, soffB = ls * 64u;
    rb[0] = read16(nb + ob);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], rb[1], acc[i][1], 0, 0, 0);
        loads_at<0>(i, cb, lt, soffA, soffB, wave, kt, ldx2, la, lb);
        __builtin_amdgcn_sched_barrier(0);
    }
    rb[1] = read16(nb + ob + 1024);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], rb[2], acc[i][2], 0, 0, 0);
        loads_at<0>(FM + i, cb, lt, soffA, soffB, wave, kt, ldx2, la, lb);
        __builtin_amdgcn_sched_barrier(0);
    }
    const lds_char* pa = (const lds_char*)(size_t)stage_addr(nb, oa);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        acc[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], rb[3], acc[i][3], 0, 0, 0);
        fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa + i * 1024));
        loads_at<0>(2 * FM + i, cb, lt, soffA, soffB, wave, kt, ldx2, la, lb);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool OUT_FP32>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_dense_kernel(Args a) {
    constexpr int SB = STAGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[NB * SB];
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    const int p = blockIdx.x;
    int Lt = tile_of(a, p, 0);
    if (Lt < 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm0 = (wave / (WAVES / 2)) * WM, wn0 = (wave % (WAVES / 2)) * 64;
    const int r = lane & 15, q = lane >> 4;
    // LDS read offsets: A fragment i of the wave at (wm0 / 16 + i) KB + 16 lane; B fragment j at token row
    // wn0 + 16 j + r, unit q (swizzled)
    const uint32_t oa = (uint32_t)((wm0 >> 4) * 1024 + lane * 16);
    const uint32_t ob = (uint32_t)(A_TILE + (wn0 + r) * 64 + 16 * (q ^ ((r >> 2) & 3)));
    // load offsets (the range-checked lane part): A 16 lane; B row lane / 4 of a 16-row group, unit lane % 4 of
    // that row's swizzled order
    const uint32_t la = (uint32_t)(16 * lane);
    const uint32_t lb = (uint32_t)((lane >> 2) * a.ldx * 2 + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
    const int S = (int)(a.K / BKD);
    const uint32_t kt = (uint32_t)S, ldx2 = (uint32_t)(a.ldx * 2);

    f32x4 acc[FM][4];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Tile cur_t = tile<OUT_FP32>(a, Lt);
    Tile nxt_t = tile<OUT_FP32>(a, tile_of(a, p, 1));
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const bool here = i < S;
        const uint32_t ls = here ? i : i - S;
        if (i == NB - 1) {
            wait_vmcnt<(NB - 2) * L>();
            __builtin_amdgcn_s_barrier();
        }
#pragma unroll
        for (int k = 0; k < L; k++) {
            const Tile& t = here ? cur_t : nxt_t;
            if (k == 0) load<0>(i * SB, t, ls * 1024u, ls * 64u, wave, kt, ldx2, la, lb);
            if (k == 1) load<1>(i * SB, t, ls * 1024u, ls * 64u, wave, kt, ldx2, la, lb);
            if (k == 2) load<2>(i * SB, t, ls * 1024u, ls * 64u, wave, kt, ldx2, la, lb);
            if (k == 3) load<3>(i * SB, t, ls * 1024u, ls * 64u, wave, kt, ldx2, la, lb);
        }
    }
    bf16x8 fa[FM], rb[4];
#pragma unroll
    for (int i = 0; i < FM; i++) fa[i] = read16(l0 + oa + i * 1024);
    rb[0] = read16(l0 + ob);
    rb[1] = read16(l0 + ob + 1024);
    uint32_t cur = 0;
    for (int k = 1;; k++) {
        int s = 0;
        for (; s < S - NB; s++) {
            const uint32_t nxt = cur == (NB - 1) * SB ? 0u : cur + SB;
            stage(l0, cur, nxt, cur_t, (uint32_t)(s + NB), acc, fa, rb, oa, ob, wave, kt, ldx2, la, lb);
            cur = nxt;
        }
        for (; s < S; s++) {
            const uint32_t nxt = cur == (NB - 1) * SB ? 0u : cur + SB;
            stage(l0, cur, nxt, nxt_t, (uint32_t)(s + NB - S), acc, fa, rb, oa, ob, wave, kt, ldx2, la, lb);
            cur = nxt;
        }
        {
            const int64_t mw = cur_t.m0 + wm0, nw = cur_t.n0 + wn0;
            if ((mw + WM <= a.M) && (nw + 64 <= a.N) && a.y_vec)
                store_tile_tm<OUT_FP32, true>(acc, a, cur_t.y, mw, nw, lane);
            else
                store_tile_tm<OUT_FP32, false>(acc, a, cur_t.y, mw, nw, lane);
        }
        if (!nxt_t.valid) break;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        cur_t = nxt_t;
        nxt_t = tile<OUT_FP32>(a, tile_of(a, p, k + 1));
    }
    wait_vmcnt<0>();
}

// Dense M x K bf16 (row pitch ldw) -> the tiled operand order above; rows past M padded with zeros. One thread
// per 16-byte chunk of the output.
__global__ __launch_bounds__(256) void dense_tile_kernel(const uint16_t* __restrict__ W, int64_t M, int64_t K, int64_t ldw,
                                                         u32x4* __restrict__ out, int64_t chunks) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t kt = K / BKD;
    const int l = (int)(c & 63);
    const int64_t t = (c >> 6) % kt, b = (c >> 6) / kt;
    const int64_t m = 16 * b + (l & 15), k = BKD * t + 8 * (l >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < M) v = *reinterpret_cast<const u32x4*>(W + m * ldw + k);
    out[c] = v;
}
}  // namespace dense_ref

}  // namespace tiled_bf16

bool gemm_bf16_tiled_ok(const GemmArgs& g) {
    // 32-bit load offsets stay below bit 31, which marks the loads past the last tile: 64 rows of X
    // (64 * ldx * 2), token-major 256 rows (256 * ldx * 2), and 16 row blocks of compressed tiles
    // (16 * K / 64 * 1 KB); 16-byte aligned rows of X in every batch entry
    const bool x_ok = g.ldx % 8 == 0 && (reinterpret_cast<uintptr_t>(g.X) & 15) == 0 && (g.batch == 1 || g.sx % 8 == 0);
    const bool tm_ok = !g.tm || (g.K % 64 == 0 && g.ldx < ((int64_t)1 << 22));
    const int64_t tiles = ((g.M + 255) / 256) * ((g.N + 127) / 128) * g.batch;
    return x_ok && tm_ok && g.N > 64 && g.ldx < ((int64_t)1 << 24) && g.K < ((int64_t)1 << 22) && tiles < (1 << 30);
}

// Number of compute units of the current device (cached per device).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Tile width for a launch of the tiled int8 GEMM (either layout). A 128-wide tile costs about C128 of
// a 256-wide one (measured on MI355X), so it wins when the 256-wide tiles leave a last partial turn that
// the 128-wide ones fill better: e.g. 3072 x 8192 has 384 tiles of 256 x 256 on 256 compute units (two
// turns), and 768 of 256 x 128 (three turns of the cheaper tile).
int tiled_tile_width(const GemmArgs& g) {
    constexpr double C128 = 0.6;
    const int64_t cus = device_cus();
    const int64_t tm = (g.M + 255) / 256;
    const int64_t t256 = tm * ((g.N + 255) / 256) * g.batch, t128 = tm * ((g.N + 127) / 128) * g.batch;
    const double c256 = (double)((t256 + cus - 1) / cus), c128 = C128 * (double)((t128 + cus - 1) / cus);
    return c128 < c256 ? 128 : 256;
}

template <bool TM, int BNT, int OCC>
static hipError_t launch_bn(const GemmArgs& g, hipStream_t s) {
    tiled_bf16::Args a;
    a.vals = static_cast<const uint16_t*>(g.values); a.meta = g.meta;
    a.X = static_cast<const uint16_t*>(g.X); a.Y = g.Y;
    a.M = g.M; a.K = g.K; a.N = g.N; a.ldx = g.ldx; a.ldy = g.ldy;
    a.sxb = g.sx; a.syb = g.sy;
    a.tilesM = (int)((g.M + tiled_bf16::BM - 1) / tiled_bf16::BM);
    a.tilesN = (int)((g.N + BNT - 1) / BNT);
    a.batch = (int)g.batch;
    // vector stores: 16-byte aligned Y rows in every batch entry, and a lane quad's row offsets in 32 bits
    const int64_t es = g.out_fp32 ? 4 : 2;
    a.y_vec = ((reinterpret_cast<uintptr_t>(g.Y) & 15) == 0) && ((g.ldy * es) % 16 == 0) &&
              (g.batch == 1 || (g.sy * es) % 16 == 0) && g.ldy * es * 16 < ((int64_t)1 << 31);
    const int T = a.tilesM * a.tilesN * a.batch;
    const int S = (int)((g.K + tiled_bf16::BK - 1) / tiled_bf16::BK);
    // workgroups walking several tiles, OCC per compute unit (the eight-wave token-major workgroup fills a CU
    // alone); one tile each when a tile has fewer stages than there are stage buffers (the cross-tile pipeline
    // then has nothing to overlap)
    if constexpr (TM) {
        using C = tiled_bf16::TmCfg<BNT>;
        const int slots = device_cus() * (BNT == 256 ? 1 : 2);
        const unsigned grid = (unsigned)(S >= C::NBUF && T > slots ? slots : T);
        if (g.out_fp32)
            hipLaunchKernelGGL((tiled_bf16::gemm_bf16_tm_kernel<true, BNT>), dim3(grid), dim3(64 * C::WAVES), 0, s, a);
        else
            hipLaunchKernelGGL((tiled_bf16::gemm_bf16_tm_kernel<false, BNT>), dim3(grid), dim3(64 * C::WAVES), 0, s, a);
    } else {
        using C = tiled_bf16::Cfg<BNT, OCC>;
        const int slots = device_cus() * OCC;
        const unsigned grid = (unsigned)(S >= C::NBUF && T > slots ? slots : T);
        if (g.out_fp32)
            hipLaunchKernelGGL((tiled_bf16::gemm_bf16_tiled_kernel<true, BNT, OCC>), dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((tiled_bf16::gemm_bf16_tiled_kernel<false, BNT, OCC>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// Configuration of a bf16 launch, measured on MI355X (bit-identical results: the K order inside a tile does
// not depend on the tile shape):
//  - from 32 stages (K >= 2048) 256 x 256 tiles, unless they would leave more than three quarters of the CUs
//    idle: a workgroup of 256 x 128 alone on its CU runs its single wave per SIMD latency-bound, and two of
//    them share the loads of a 256 x 256 tile less well (token-major, against the rule below: 28672 x 8192 x
//    512 144.8 -> 128.0 us, 11008 x 4096 x 1024 58.0 -> 53.1, 3072 x 4096 x 6304 106.5 -> 100.3, 16384 x 8192
//    x 512 113.7 -> 108.6, 768 x 3072 x 8192 32.9 either way; feature-major 28672 x 8192 x 512 146.2 -> 143.7);
//  - below that, 256 x 128 tiles with two workgroups per CU fill the CUs better when there are fewer 256 x 256 tiles
//    than CUs, and fill a partial last turn better: their last turn's tiles run one per CU, at about 0.6
//    of a paired turn, while a full turn of 256 x 256 tiles costs about 0.92 of one (3072 x 768 x 6304
//    token-major: 26.4 us against 30.8 with 256 x 256);
//  - 256 x 256 tiles otherwise (a full first turn, or more than two turns): token-major with eight waves per
//    workgroup, two per SIMD, so the big tile's re-use stays and a second wave covers each one's barrier
//    and load waits (11008 x 4096 x 4096: 235.4 -> 212.2 us against four waves; 28672 x 8192 x 8192:
//    2115 -> 1986 us; against 256 x 128 two per CU: 4096^3 90.8 -> 83.7 us, 4096 x 4096 x 8192 160 -> 152,
//    4096 x 2048 x 8192 101 -> 91); feature-major with four waves (its eight-wave build spills registers;
//    4096^3 82.4 -> 77.7 us).
hipError_t launch_gemm_bf16_tiled(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ((g.M + 255) / 256) * g.batch, cus = device_cus();
    const int64_t t256 = tm * ((g.N + 255) / 256), t128 = tm * ((g.N + 127) / 128);
    // turns of each tiling in units of a paired 256 x 128 turn
    const double c256 = 0.92 * (double)((t256 + cus - 1) / cus);
    const int64_t rem = t128 % (2 * cus);
    const double c128 = (double)(t128 / (2 * cus)) + (rem == 0 ? 0.0 : rem <= cus ? 0.6 : 1.0);
    const int64_t stages = (g.K + tiled_bf16::BK - 1) / tiled_bf16::BK;
    if (stages >= 32 && 4 * t256 >= cus)
        return g.tm ? launch_bn<true, 256, 1>(g, s) : launch_bn<false, 256, 1>(g, s);
    if (t256 < cus || (t256 <= 2 * cus && c128 <= c256))
        return g.tm ? launch_bn<true, 128, 2>(g, s) : launch_bn<false, 128, 2>(g, s);
    return g.tm ? launch_bn<true, 256, 1>(g, s) : launch_bn<false, 256, 1>(g, s);
}

}  // namespace sp24

namespace sp24 {

// Host side of the dense reference (measurement only; arguments validated by the C ABI).
hipError_t launch_dense_tile(const void* W, int64_t M, int64_t K, int64_t ldw, void* Wt, hipStream_t s) {
    const int64_t chunks = (M + 15) / 16 * (K / tiled_bf16::dense_ref::BKD) * 64;
    hipLaunchKernelGGL(tiled_bf16::dense_ref::dense_tile_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(W), M, K, ldw, static_cast<u32x4*>(Wt), chunks);
    return hipGetLastError();
}

hipError_t launch_gemm_dense_ref(const GemmArgs& g, hipStream_t s) {
    namespace D = tiled_bf16::dense_ref;
    tiled_bf16::Args a;
    a.vals = static_cast<const uint16_t*>(g.values); a.meta = nullptr;
    a.X = static_cast<const uint16_t*>(g.X); a.Y = g.Y;
    a.M = g.M; a.K = g.K; a.N = g.N; a.ldx = g.ldx; a.ldy = g.ldy;
    a.sxb = 0; a.syb = 0;
    a.tilesM = (int)((g.M + tiled_bf16::BM - 1) / tiled_bf16::BM);
    a.tilesN = (int)((g.N + D::BN - 1) / D::BN);
    a.batch = 1;
    const int64_t es = g.out_fp32 ? 4 : 2;
    a.y_vec = ((reinterpret_cast<uintptr_t>(g.Y) & 15) == 0) && ((g.ldy * es) % 16 == 0) && g.ldy * es * 16 < ((int64_t)1 << 31);
    const int T = a.tilesM * a.tilesN;
    const int S = (int)(g.K / D::BKD);
    const int slots = device_cus();
    const unsigned grid = (unsigned)(S >= D::NB && T > slots ? slots : T);
    if (g.out_fp32)
        hipLaunchKernelGGL((D::gemm_dense_kernel<true>), dim3(grid), dim3(64 * D::WAVES), 0, s, a);
    else
        hipLaunchKernelGGL((D::gemm_dense_kernel<false>), dim3(grid), dim3(64 * D::WAVES), 0, s, a);
    return hipGetLastError();
}

}  // namespace sp24
