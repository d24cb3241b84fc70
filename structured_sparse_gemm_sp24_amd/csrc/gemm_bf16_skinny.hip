// Sparse x dense GEMM for few tokens (N <= 64), bf16 in, fp32 accumulate (NVIDIA blog on Ampere
// structured sparsity, Figure 1; Orin NN design, Chapter 7, section 2.1 Step 3).
//
// With N this small the product is bound by streaming the compressed weight (1.125 bytes per dense
// weight) from HBM once; X is a few KB to a few MB and stays in L2. So the kernel is built to keep
// many weight bytes in flight and to touch each weight byte once:
//  - a workgroup owns R consecutive 16-row blocks of the weight and all N columns (NF fragments of
//    16 columns); its S waves split the K tiles of those blocks into S contiguous ranges;
//  - a wave walks its range U tiles at a time, double-buffered: the next round's compressed tiles
//    (one 16-byte value load and one 2-byte index load per lane and block, in smfmac lane order) and
//    X fragments are requested before the current round's smfmacs;
//  - the X fragments of a tile (lane = column, 16 k values) are built once per tile and shared by the
//    R blocks. Feature-major X (K x N): for a unit-pitch vector (N = 1) from two 16-byte loads; when
//    rows of X are 16-byte aligned and N is a multiple of 8, by staging the 64 x 16 NF tile through a
//    wave-private LDS slot (16-byte loads, ds_write_b128, then ds_read_b64_tr_b16); otherwise element
//    by element. Token-major X (N x K): a lane's 16 k values are two runs of 8 consecutive elements of
//    its token's row, so two 16-byte loads when rows are 16-byte aligned (element loads in the K tail
//    tile and otherwise);
//  - at the end the S partial 16 x 16 accumulators of each block are summed through LDS in wave order
//    (deterministic), rounded if the output is bf16, and stored with bounds checks (M x N or, token-
//    major, N x M).
// A batch of independent products sharing the weight (1x1 conv over B images) is grid dimension y.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace skinny {

struct Args {
    const uint16_t* vals;
    const uint8_t* meta;
    int64_t M, K, N;
    const uint16_t* X;
    int64_t ldx, sxb;
    void* Y;
    int64_t ldy, syb;
    int out_fp32;
};

// X fragment for columns 16 f .. 16 f + 15 of tile k0 (smfmac B operand: lane n = r holds
// k = k0 + 8q + (e & 7) + 32 (e >> 3)); zero past K and past N. The general case reads single
// elements through a buffer descriptor covering exactly X's extent, so rows past K come back as 0.
template <bool UNIT>
__device__ __forceinline__ bf16x16 load_x(const uint16_t* __restrict__ X, __amdgpu_buffer_rsrc_t rx, int64_t ldx,
                                          int64_t K, int64_t N, int64_t k0, int64_t n, int q) {
    u32x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n < N) {
        if (UNIT) {
            // N == 1 with unit pitch: the 16 values are two runs of 8 consecutive elements
            const int64_t ka = k0 + 8 * q, kb = ka + 32;
            if (kb + 8 <= K) {
                const u32x4 lo = *reinterpret_cast<const u32x4*>(X + ka);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(X + kb);
                b = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const int64_t k = k0 + 8 * q + (e & 7) + 32 * (e >> 3);
                    const uint32_t v0 = k < K ? X[k] : 0u;
                    const uint32_t v1 = k + 1 < K ? X[k + 1] : 0u;
                    b[e >> 1] = v0 | (v1 << 16);
                }
            }
        } else {
            const uint32_t ld2 = (uint32_t)ldx * 2;
            const uint32_t o = (uint32_t)(((k0 + 8 * q) * ldx + n) * 2);
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const uint32_t oe = o + (uint32_t)((e & 7) + 32 * (e >> 3)) * ld2;
                const uint32_t v0 = __builtin_amdgcn_raw_buffer_load_b16(rx, (int)oe, 0, 0);
                const uint32_t v1 = __builtin_amdgcn_raw_buffer_load_b16(rx, (int)(oe + ld2), 0, 0);
                b[e >> 1] = v0 | (v1 << 16);
            }
        }
    }
    return __builtin_bit_cast(bf16x16, b);
}

// Token-major X (row n holds token n's K values): lane n = r's fragment is the two runs
// k0 + 8q .. +7 and k0 + 32 + 8q .. +7 of its row. VEC: 16-byte loads (rows 16-byte aligned) except in
// the K tail tile, where elements at k >= K (the next row, or row padding) must read as zero.
template <bool VEC>
__device__ __forceinline__ bf16x16 load_x_tm(__amdgpu_buffer_rsrc_t rx, int64_t ldx, int64_t K, int64_t N, int64_t k0,
                                             int64_t n, int q) {
    u32x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n < N) {
        const uint32_t o = (uint32_t)((n * ldx + k0 + 8 * q) * 2);
        if (VEC && k0 + 64 <= K) {
            const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o, 0, 0));
            const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(o + 64), 0, 0));
            b = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const int d = (e & 7) + 32 * (e >> 3);
                const int64_t k = k0 + 8 * q + d;
                const uint32_t v0 = k < K ? __builtin_amdgcn_raw_buffer_load_b16(rx, (int)(o + 2 * d), 0, 0) : 0u;
                const uint32_t v1 = k + 1 < K ? __builtin_amdgcn_raw_buffer_load_b16(rx, (int)(o + 2 * d + 2), 0, 0) : 0u;
                b[e >> 1] = v0 | (v1 << 16);
            }
        }
    }
    return __builtin_bit_cast(bf16x16, b);
}

enum { X_ELEMENTS = 0, X_UNIT_VECTOR = 1, X_STAGED = 2, X_TOKEN = 3, X_TOKEN_ELEMENTS = 4 };

// Staged X tile (64 rows x 16 NF bf16) in a wave's LDS slot: row pitch P = 32 NF bytes plus a gap of
// G bytes after every 8 rows. The gap puts the 16 rows x 32 bytes of each transposing read (rows
// 8q + {0..3}, q = 0..3) into 8 distinct 32-byte bank groups, and every read of a fragment is then
// one lane address plus immediates (+4 rows, +32 rows) -- checked by enumeration for NF = 1, 2, 4.
template <int NF>
struct XTile {
    static constexpr int P = 32 * NF;
    static constexpr int G = NF == 1 ? 64 : 32;
    static constexpr int GROUP = 8 * P + G;
    static constexpr int BYTES = 8 * GROUP;
    static constexpr __device__ int row(int k) { return (k >> 3) * GROUP + (k & 7) * P; }
};

template <int NF, int R, int U, int XMODE>
struct Round {
    u32x4 a[U][R];
    uint32_t idx[U][R];
    bf16x16 b[U][NF];
    u32x4 xs[XMODE == X_STAGED ? U : 1][2 * NF];  // staged X chunks (16 bytes each) of every tile
};

template <int NF, int R, int S, int U, int XMODE>
__global__ __launch_bounds__(64 * S) void gemm_bf16_skinny(Args g) {
    constexpr bool TM = XMODE == X_TOKEN || XMODE == X_TOKEN_ELEMENTS;
    const uint8_t* __restrict__ meta = g.meta;
    const uint16_t* __restrict__ vals = g.vals;
    const int64_t M = g.M, K = g.K, N = g.N, ldx = g.ldx, ldy = g.ldy;
    const int out_fp32 = g.out_fp32;
    const uint16_t* __restrict__ X = g.X + (int64_t)blockIdx.y * g.sxb;
    char* const Y = static_cast<char*>(g.Y) + (int64_t)blockIdx.y * g.syb * (out_fp32 ? 4 : 2);
    // the wave-private X slots during the K loop, the reduction buffer after it
    constexpr int RED_BYTES = S * R * NF * 256 * 4;
    constexpr int X_BYTES = XMODE == X_STAGED ? S * XTile<NF>::BYTES : 0;
    __shared__ __attribute__((aligned(16))) char smem[RED_BYTES > X_BYTES ? RED_BYTES : X_BYTES];
    float* const red = reinterpret_cast<float*>(smem);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int64_t nblocks = (M + 15) / 16;
    const int64_t b0 = (int64_t)blockIdx.x * R;
    const int64_t T = (K + 63) / 64;  // compressed tiles per row block
    const int64_t t0 = T * wave / S, t1 = T * (wave + 1) / S;
    int nb = (int)(nblocks - b0 < R ? nblocks - b0 : R);

    // tile (b, t): values at ((b * T + t) * 64 + lane) * 16 bytes, index at ((b * T + t) * 64 + lane) * 2
    const u32x4* vt = reinterpret_cast<const u32x4*>(vals) + b0 * T * 64 + lane;
    const uint16_t* mt = reinterpret_cast<const uint16_t*>(meta) + b0 * T * 64 + lane;
    // X's extent in bytes: (K - 1) rows of pitch ldx plus N elements, token-major (N - 1) rows plus K
    // (below 2^31, checked on the host), rounded up to a whole dword (the range check passes a dword
    // only if all of it is in range; the rounding stays inside the aligned dword that holds the last
    // element)
    const int64_t x_elems = TM ? (N - 1) * ldx + K : (K - 1) * ldx + N;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)((x_elems * 2 + 3) & ~3), 0x00020000);

    f32x4 acc[R][NF];
#pragma unroll
    for (int j = 0; j < R; j++)
#pragma unroll
        for (int f = 0; f < NF; f++) acc[j][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    char* const xslot = smem + wave * XTile<NF>::BYTES;
    // lane address of the transposing reads of fragment f (t = 0): row 8q + r/4, columns 16 f + 4 (r % 4)
    const int xrd = XTile<NF>::row(8 * q + (r >> 2)) + 2 * (4 * (r & 3));

    auto issue = [&](Round<NF, R, U, XMODE>& rd, int64_t t) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t tt = t + u;
            const bool ok = tt < t1;
#pragma unroll
            for (int j = 0; j < R; j++) {
                if (ok && j < nb) {
                    rd.a[u][j] = __builtin_nontemporal_load(vt + (j * T + tt) * 64);
                    rd.idx[u][j] = __builtin_nontemporal_load(mt + (j * T + tt) * 64);
                } else {
                    rd.a[u][j] = u32x4{0, 0, 0, 0};
                    rd.idx[u][j] = 0x4444u;
                }
            }
            if constexpr (XMODE == X_STAGED) {
                // chunk c = lane + 64 i of the tile: row c / (2 NF), 8 columns at 8 (c % (2 NF)); chunks
                // wholly past N (N is a multiple of 8 here) reread the row's first chunk, rows past K
                // are out of the descriptor's range and read as zeros
#pragma unroll
                for (int i = 0; i < 2 * NF; i++) {
                    const int c = lane + 64 * i, row = c / (2 * NF), col = 8 * (c % (2 * NF));
                    const int64_t k = 64 * tt + row;
                    const uint32_t off = (uint32_t)((k * ldx + (col < N ? col : 0)) * 2);
                    rd.xs[u][i] = ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0))
                                     : u32x4{0, 0, 0, 0};
                }
            } else {
#pragma unroll
                for (int f = 0; f < NF; f++) {
                    if (ok && TM)
                        rd.b[u][f] = load_x_tm<XMODE == X_TOKEN>(rx, ldx, K, N, 64 * tt, 16 * f + r, q);
                    else if (ok)
                        rd.b[u][f] = load_x<XMODE == X_UNIT_VECTOR>(X, rx, ldx, K, N, 64 * tt, 16 * f + r, q);
                    else
                        rd.b[u][f] = __builtin_bit_cast(bf16x16, u32x8{0, 0, 0, 0, 0, 0, 0, 0});
                }
            }
        }
    };
    auto compute = [&](Round<NF, R, U, XMODE>& rd) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if constexpr (XMODE == X_STAGED) {
                // write the tile into the slot (the previous tile's reads of it have completed: their
                // results fed the previous smfmacs), then read the NF fragments back transposed
#pragma unroll
                for (int i = 0; i < 2 * NF; i++) {
                    const int c = lane + 64 * i, row = c / (2 * NF), col = 8 * (c % (2 * NF));
                    *reinterpret_cast<u32x4*>(xslot + XTile<NF>::row(row) + 2 * col) = rd.xs[u][i];
                }
#pragma unroll
                for (int f = 0; f < NF; f++) {
                    u32x8 b;
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        const int imm = XTile<NF>::row(4 * (t & 1) + 32 * (t >> 1)) + 32 * f;
                        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(xslot + xrd + imm));
                        b[2 * t] = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                        b[2 * t + 1] = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
                    }
                    rd.b[u][f] = __builtin_bit_cast(bf16x16, b);
                }
            }
#pragma unroll
            for (int j = 0; j < R; j++)
#pragma unroll
                for (int f = 0; f < NF; f++)
                    acc[j][f] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, rd.a[u][j]),
                                                                          rd.b[u][f], acc[j][f], (int)rd.idx[u][j], 0,
                                                                          0);
        }
    };

    if (t0 < t1) {
        Round<NF, R, U, XMODE> cur, nxt;
        issue(cur, t0);
        int64_t t = t0;
        for (; t + U < t1; t += U) {
            issue(nxt, t + U);
            compute(cur);
            cur = nxt;
        }
        compute(cur);
    }

    // sum the S partial tiles of each block in wave order
    if constexpr (XMODE == X_STAGED) __syncthreads();  // the X slots become the reduction buffer
#pragma unroll
    for (int j = 0; j < R; j++)
#pragma unroll
        for (int f = 0; f < NF; f++)
#pragma unroll
            for (int i = 0; i < 4; i++) red[((wave * R + j) * NF + f) * 256 + (4 * q + i) * 16 + r] = acc[j][f][i];
    __syncthreads();
    for (int e = threadIdx.x; e < R * NF * 256; e += 64 * S) {
        // consecutive threads take consecutive elements of an output row: columns of Y (M x N), or rows
        // of the block (token-major, N x M)
        const int j = e / (NF * 256), f = (e / 256) % NF;
        const int row = TM ? e % 16 : (e / 16) % 16, col = TM ? (e / 16) % 16 : e % 16;
        float s = 0.f;
#pragma unroll 4
        for (int w = 0; w < S; w++) s += red[((w * R + j) * NF + f) * 256 + row * 16 + col];
        const int64_t m = (b0 + j) * 16 + row, n = 16 * f + col;
        if (j < nb && m < M && n < N) {
            const int64_t o = TM ? n * ldy + m : m * ldy + n;
            if (out_fp32)
                reinterpret_cast<float*>(Y)[o] = s;
            else
                reinterpret_cast<uint16_t*>(Y)[o] = f32_to_bf16_rne(s);
        }
    }
}

template <int NF, int R, int S, int U>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
    Args a;
    a.vals = static_cast<const uint16_t*>(g.values);
    a.meta = g.meta;
    a.M = g.M; a.K = g.K; a.N = g.N;
    a.X = static_cast<const uint16_t*>(g.X);
    a.ldx = g.ldx; a.sxb = g.sx;
    a.Y = g.Y;
    a.ldy = g.ldy; a.syb = g.sy;
    a.out_fp32 = g.out_fp32;
    const unsigned grid = (unsigned)(((g.M + 15) / 16 + R - 1) / R);
    // grid y covers at most 65535 batch entries per launch
    for (int64_t b0 = 0; b0 < g.batch; b0 += 65535) {
        const unsigned gb = (unsigned)(g.batch - b0 < 65535 ? g.batch - b0 : 65535);
        Args e = a;
        e.X = a.X + b0 * a.sxb;
        e.Y = static_cast<char*>(a.Y) + b0 * a.syb * (g.out_fp32 ? 4 : 2);
        const dim3 grd(grid, gb), blk(64 * S);
        if (g.tm) {
            if (g.ldx % 8 == 0)
                hipLaunchKernelGGL((gemm_bf16_skinny<NF, R, S, U, X_TOKEN>), grd, blk, 0, s, e);
            else
                hipLaunchKernelGGL((gemm_bf16_skinny<NF, R, S, U, X_TOKEN_ELEMENTS>), grd, blk, 0, s, e);
        } else if (NF == 1 && g.N == 1 && g.ldx == 1) {
            hipLaunchKernelGGL((gemm_bf16_skinny<NF, R, S, U, X_UNIT_VECTOR>), grd, blk, 0, s, e);
        } else if (g.ldx % 8 == 0 && g.N % 8 == 0) {
            hipLaunchKernelGGL((gemm_bf16_skinny<NF, R, S, U, X_STAGED>), grd, blk, 0, s, e);
        } else {
            hipLaunchKernelGGL((gemm_bf16_skinny<NF, R, S, U, X_ELEMENTS>), grd, blk, 0, s, e);
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace skinny

bool gemm_bf16_skinny_ok(const GemmArgs& g) {
    // 32-bit byte offsets for every element the tiles touch (K padded to 64, plus one tile)
    const int64_t extent = g.tm ? g.N * g.ldx + g.K + 128 : (g.K + 128) * g.ldx;
    return g.N <= 64 && extent * 2 < ((int64_t)1 << 31);
}

// Row blocks per workgroup (R), waves per workgroup (S) and tiles per round (U) by size: about 256 or
// more workgroups, R as large as that allows (each X fragment is then shared by more weight tiles);
// the unit-vector case reads its X fragment cheaply and prefers more, smaller workgroups. Chosen by
// measurement on MI355X over R in {1, 2, 4}, S in {4, 8, 16}, U in {1, 2, 4}.
// Token-major X with 17 or more tokens (and 9-16 tokens past 256 row blocks, where the LDS-ring kernel
// is not used): measured over R in {1, ..., 8}, S in {4, 8, 16}, U in {1, 2} with weight copies rotated
// beyond the Infinity Cache. The best grid is one round that loads every CU alike: past 512 row blocks, R =
// ceil(blocks / CUs), which gives each CU R or R - 1 blocks (a power of two R left up to a quarter of the CUs
// idle: 11008 x 4096 at N = 16 / 32 / 64 13.9 / 16.8 / 25.4 -> 12.2 / 14.8 / 23.8 us with R = 3 instead of 4,
// 8200 x 4096 at N = 16 / 48 12.8 / 22.9 -> 11.7 / 21.0, 28672 x 8192 at N = 32 / 64 53.3 / 70.4 -> 49.8 /
// 66.4 with R = 7 instead of 8; at N = 16 that weight streams at its read floor either way). For one
// fragment from 1024 row blocks, workgroups of two blocks and four waves, several per CU, are kept where
// they load the CUs as evenly (16384 x 4096: 16.0 us against 18.0 with R = 4; 20480 x 4096, 640 of them:
// 20.7 against 19.6 with R = 5).
template <int NF, int S, int U>
static hipError_t launch_r(const GemmArgs& g, hipStream_t s, int64_t r) {
    switch (r) {
    case 1: return skinny::launch<NF, 1, S, U>(g, s);
    case 2: return skinny::launch<NF, 2, S, U>(g, s);
    case 3: return skinny::launch<NF, 3, S, U>(g, s);
    case 4: return skinny::launch<NF, 4, S, U>(g, s);
    case 5: return skinny::launch<NF, 5, S, U>(g, s);
    case 6: return skinny::launch<NF, 6, S, U>(g, s);
    case 7: return skinny::launch<NF, 7, S, U>(g, s);
    default: return skinny::launch<NF, 8, S, U>(g, s);
    }
}

static hipError_t launch_skinny_tm(const GemmArgs& g, hipStream_t s, int64_t nb) {
    const int64_t cus = device_cus();
    const int64_t r = (nb + cus - 1) / cus;  // blocks per workgroup for a one-round grid (R <= 8 below)
    if (g.N <= 16) {
        if (nb > 8 * cus) return skinny::launch<1, 8, 8, 1>(g, s);
        if (nb > 6 * cus) return launch_r<1, 8, 1>(g, s, r);
        if (nb >= 1024) {
            // workgroups of two blocks: the most blocks a CU gets is 2 ceil(ceil(nb / 2) / CUs)
            const int64_t pairs = 2 * (((nb + 1) / 2 + cus - 1) / cus);
            return pairs <= r ? skinny::launch<1, 2, 4, 1>(g, s) : launch_r<1, 4, 1>(g, s, r);
        }
        return nb > 512 ? launch_r<1, 4, 2>(g, s, r) : skinny::launch<1, 2, 8, 2>(g, s);
    }
    if (g.N <= 32) {
        if (nb > 512) return r <= 8 ? launch_r<2, 8, 1>(g, s, r) : skinny::launch<2, 8, 8, 1>(g, s);
        if (nb > 256) return skinny::launch<2, 2, 8, 1>(g, s);
        return nb >= 192 ? skinny::launch<2, 1, 8, 1>(g, s) : skinny::launch<2, 1, 16, 1>(g, s);
    }
    if (nb > 512) return r <= 8 ? launch_r<4, 4, 1>(g, s, r) : skinny::launch<4, 8, 4, 1>(g, s);
    if (nb > 256) return skinny::launch<4, 2, 8, 1>(g, s);
    return skinny::launch<4, 1, 8, 1>(g, s);
}

hipError_t launch_gemm_bf16_skinny(const GemmArgs& g, hipStream_t s) {
    const int64_t nb = (g.M + 15) / 16;
    const bool vec1 = g.N == 1 && (g.tm || g.ldx == 1);  // one token: X is a contiguous K-vector
    if (vec1) {
        if (nb >= 1024) return skinny::launch<1, 4, 16, 1>(g, s);
        if (nb >= 512) return skinny::launch<1, 2, 4, 2>(g, s);
        return skinny::launch<1, 1, 8, 4>(g, s);
    }
    if (g.tm && (g.N > 16 || nb > 256)) return launch_skinny_tm(g, s, nb);
    if (g.N <= 16) {
        if (nb >= 512) return skinny::launch<1, 4, 16, 1>(g, s);
        return skinny::launch<1, 1, 16, 2>(g, s);
    }
    if (g.N <= 32) {
        if (nb >= 1024) return skinny::launch<2, 4, 8, 1>(g, s);
        if (nb >= 512) return skinny::launch<2, 2, 16, 1>(g, s);
        return skinny::launch<2, 1, 16, 1>(g, s);
    }
    if (nb >= 1024) return skinny::launch<4, 4, 8, 1>(g, s);
    if (nb >= 512) return skinny::launch<4, 2, 8, 1>(g, s);
    return skinny::launch<4, 1, 8, 1>(g, s);
}

}  // namespace sp24
