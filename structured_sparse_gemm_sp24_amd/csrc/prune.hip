// 2:4 prune + compress, and decompress (Orin NN design, Chapter 7, section 2.1 Steps 1-2; NVIDIA
// blog on Ampere structured sparsity, Figure 1).
//
// Both kernels are HBM streams. Prune/compress is organized by compressed tile (16 rows x 64 bytes
// of values, in the lane order of the sparse MFMA operand): lane l of a wave owns slot l of a tile,
// i.e. row l % 16 and dense columns [KT/4 * (l / 16), +KT/4) of the tile (KT = 128 / value size).
// It loads those columns (16-byte loads; several tiles per lane in flight), scores and selects in
// registers, and writes its 16 value bytes and 4 / value-size metadata bytes, so every wave writes
// whole 1 KB value tiles and whole metadata tiles with contiguous stores. Decompress keeps one thread
// per 16-column chunk of a row.
//
// Selection is a knockout over the group: (0 vs 1) and (2 vs 3), then the two winners; the
// runner-up is the better of the two elements that lost directly to the champion. "a beats b" for
// a < b is key[a] >= key[b], i.e. larger score wins and equal scores go to the lower index.
// Magnitude keys are the sign-cleared bit patterns (integer order equals |w| order for finite IEEE
// values) or |q| for int8; Wanda keys are the bits of the fp32 product fl32(|w|) * norms[k].
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {

enum { DT_BF16 = 0, DT_FP16 = 1, DT_FP32 = 2, DT_I8 = 3 };

// Storage type of one weight element (bit pattern).
template <int DT> struct Elem { typedef uint16_t T; };
template <> struct Elem<DT_FP32> { typedef uint32_t T; };
template <> struct Elem<DT_I8> { typedef uint8_t T; };

// v[i] for i in 0..3 by selects (a register array indexed at run time would go to scratch).
template <typename T>
__device__ __forceinline__ T pick4(T v0, T v1, T v2, T v3, int i) {
    return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
}

// Kept positions (lo < hi) of the group whose keys are k[0..3].
__device__ __forceinline__ void knockout_top2(const uint32_t k[4], int& lo, int& hi) {
    const bool a01 = k[0] >= k[1], a23 = k[2] >= k[3];
    const int w1 = a01 ? 0 : 1, l1 = a01 ? 1 : 0;  // winner / loser of the first match
    const int w2 = a23 ? 2 : 3, l2 = a23 ? 3 : 2;
    const uint32_t kw1 = a01 ? k[0] : k[1], kw2 = a23 ? k[2] : k[3];
    const uint32_t kl1 = a01 ? k[1] : k[0], kl2 = a23 ? k[3] : k[2];
    int champ, second;
    if (kw1 >= kw2) {  // w1 < w2 always: ties go to w1
        champ = w1;
        second = (kl1 >= kw2) ? l1 : w2;  // l1 < w2
    } else {
        champ = w2;
        second = (kw1 >= kl2) ? w1 : l2;  // w1 < l2
    }
    lo = champ < second ? champ : second;
    hi = champ < second ? second : champ;
}

template <int DT> constexpr int esize() { return DT == DT_FP32 ? 4 : (DT == DT_I8 ? 1 : 2); }

// Selection key of one element (bit pattern v of type DT): larger key = larger score. Magnitude: the
// sign-cleared bits (IEEE) or |q| (int8); Wanda: the bits of fl32(|w|) * norm.
template <int DT, bool WANDA, typename T>
__device__ __forceinline__ uint32_t select_key(T v, float norm) {
    if (WANDA) {
        float a;
        if (DT == DT_FP32) a = __uint_as_float((uint32_t)v & 0x7FFFFFFFu);
        else if (DT == DT_FP16) a = f16_to_f32((uint16_t)(v & 0x7FFFu));
        else a = bf16_to_f32((uint16_t)(v & 0x7FFFu));
        return __float_as_uint(__fmul_rn(a, norm)) & 0x7FFFFFFFu;
    } else if (DT == DT_I8) {
        const int sv = (int)(int8_t)v;
        return (uint32_t)(sv < 0 ? -sv : sv);
    } else {
        return (uint32_t)v & (DT == DT_FP32 ? 0x7FFFFFFFu : 0x7FFFu);
    }
}

// Workgroup = 4 waves x TPW tiles of one 16-row block: wave w takes tiles t0 + w + 4 i, i < TPW.
// Slots outside the M x K weight write the padding (values 0, metadata nibbles 0x4).
template <int DT, int VOUT, bool WANDA, int TPW>
__global__ __launch_bounds__(256) void prune_compress_kernel(const void* __restrict__ W, int64_t ldw, int64_t M,
                                                             int64_t K, int64_t tiles, int64_t groups_x,
                                                             const float* __restrict__ norms, void* __restrict__ values,
                                                             uint8_t* __restrict__ meta) {
    constexpr int isz = esize<DT>(), vsz = esize<VOUT>();
    constexpr int KT = 128 / vsz;       // dense columns per tile
    constexpr int SPAN = KT / 4;        // dense columns per lane: 16 (2-byte values), 32 (int8), 8 (fp32)
    constexpr int NG = SPAN / 4;        // groups per lane
    constexpr int MB = 4 / vsz;         // metadata bytes per lane
    typedef typename Elem<DT>::T T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, qq = lane >> 4;
    const int64_t b = blockIdx.x / groups_x;
    const int64_t tx = blockIdx.x - b * groups_x;
    const int64_t row = 16 * b + r;
    const bool row_ok = row < M;
    const char* wrow = reinterpret_cast<const char*>(W) + row * ldw * isz;

    // load every tile first (TPW x SPAN elements per lane), and with Wanda the norms of the lane's span in
    // the same round: loaded inside the group loop instead, they cost a second memory round trip per wave
    // (11008 x 4096 bf16 Wanda: 33.4 us against 29.4 for magnitude)
    T x[TPW][SPAN];
    f32x4 nrm[TPW][WANDA ? NG : 1];
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int64_t t = tx * 4 * TPW + wave + 4 * i;
        const int64_t c0 = t * KT + SPAN * qq;
        if constexpr (WANDA) {
            // the span starts at a multiple of SPAN (8 or 16, which divides K), so when it starts inside K all
            // of it is inside K; norms is 16-byte aligned (checked on the host): NG 16-byte loads
#pragma unroll
            for (int g = 0; g < NG; g++)
                nrm[i][g] = (t < tiles && c0 < K) ? *reinterpret_cast<const f32x4*>(norms + c0 + 4 * g)
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int h = 0; h < (SPAN * isz) / 16; h++) {  // 16-byte pieces of the lane's span
            constexpr int PER = 16 / isz;                // elements per piece
            const int64_t c = c0 + PER * h;
            u32x4 v = u32x4{0, 0, 0, 0};
            if (row_ok && t < tiles && c < K) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + c * isz));
#pragma unroll
            for (int e = 0; e < PER; e++) {
                if (isz == 4) x[i][PER * h + e] = (T)v[e];
                if (isz == 2) x[i][PER * h + e] = (T)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                if (isz == 1) x[i][PER * h + e] = (T)((v[e >> 2] >> (8 * (e & 3))) & 0xFFu);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int64_t t = tx * 4 * TPW + wave + 4 * i;
        if (t >= tiles) break;
        const int64_t c0 = t * KT + SPAN * qq;
        T kept[2 * NG];
        uint32_t mbits = 0;
#pragma unroll
        for (int g = 0; g < NG; g++) {
            const int64_t c = c0 + 4 * g;
            if (row_ok && c < K) {
                uint32_t key[4];
                float nv[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (WANDA) {
                    nv[0] = nrm[i][g][0]; nv[1] = nrm[i][g][1]; nv[2] = nrm[i][g][2]; nv[3] = nrm[i][g][3];
                }
#pragma unroll
                for (int e = 0; e < 4; e++) key[e] = select_key<DT, WANDA>(x[i][4 * g + e], nv[e]);
                int lo, hi;
                knockout_top2(key, lo, hi);
                mbits |= (uint32_t)(lo | (hi << 2)) << (4 * g);
                kept[2 * g] = pick4(x[i][4 * g], x[i][4 * g + 1], x[i][4 * g + 2], x[i][4 * g + 3], lo);
                kept[2 * g + 1] = pick4(x[i][4 * g], x[i][4 * g + 1], x[i][4 * g + 2], x[i][4 * g + 3], hi);
            } else {
                mbits |= 0x4u << (4 * g);
                kept[2 * g] = 0;
                kept[2 * g + 1] = 0;
            }
        }
        // values: this lane's 16 bytes of tile (b, t); metadata: its MB bytes of the metadata tile
        char* vt = reinterpret_cast<char*>(values) + (b * tiles + t) * 1024 + 16 * lane;
        uint8_t* mt = meta + (b * tiles + t) * (64 * MB) + MB * lane;
        if (VOUT == DT_FP32) {
            *reinterpret_cast<uint4*>(vt) = make_uint4(kept[0], kept[1], kept[2], kept[3]);
        } else if (VOUT == DT_I8) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; k++)
                w[k] = (uint32_t)(uint8_t)kept[4 * k] | ((uint32_t)(uint8_t)kept[4 * k + 1] << 8) |
                       ((uint32_t)(uint8_t)kept[4 * k + 2] << 16) | ((uint32_t)(uint8_t)kept[4 * k + 3] << 24);
            *reinterpret_cast<uint4*>(vt) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {  // 16-bit values: bf16/fp16 bit copies, or fp32 rounded to bf16
            uint32_t h[8];
#pragma unroll
            for (int k = 0; k < 8; k++)
                h[k] = DT == DT_FP32 ? (uint32_t)f32_to_bf16_rne(__uint_as_float((uint32_t)kept[k])) : (uint32_t)kept[k];
            *reinterpret_cast<uint4*>(vt) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        }
        if (MB == 4) *reinterpret_cast<uint32_t*>(mt) = mbits;
        else if (MB == 2) *reinterpret_cast<uint16_t*>(mt) = (uint16_t)mbits;
        else *mt = (uint8_t)mbits;
    }
}

// int8 magnitude selection, two groups at a time, the group's four weights being one 32-bit word. Each byte
// becomes |q| without crossing into its neighbour (for q < 0, ~q + 1 <= 0x80). The key of position e,
// (|q| << 2) | (3 - e), is unique within the group and orders as |q| with the lower position first on ties;
// the two groups' keys of one position share a word, one per 16-bit half, and the packed 16-bit max / min
// take both groups' comparisons at once. The kept pair is the largest and second largest key: the second
// largest of four is the larger of the median of the first three and the smaller of their maximum and the
// fourth. Returns, per half, the lower (lo) and higher (hi) kept position.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t min_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t abs_i8x4(uint32_t w) {
    const uint32_t hb = w & 0x80808080u, sgn = hb >> 7;
    return (w ^ ((hb << 1) - sgn)) + sgn;  // (hb << 1) - sgn: 0xFF in each negative byte
}

__device__ __forceinline__ void top2_i8_pair(uint32_t w0, uint32_t w1, uint32_t& lo, uint32_t& hi) {
    const uint32_t a0 = abs_i8x4(w0), a1 = abs_i8x4(w1);
    // byte e of a0 into the low half, of a1 into the high half (selector bytes 0-3: a0, 4-7: a1, 0x0c: zero);
    // |q| <= 0x80, so the shift stays inside each half
    const uint32_t k0 = (__builtin_amdgcn_perm(a1, a0, 0x0c040c00u) << 2) | 0x00030003u;
    const uint32_t k1 = (__builtin_amdgcn_perm(a1, a0, 0x0c050c01u) << 2) | 0x00020002u;
    const uint32_t k2 = (__builtin_amdgcn_perm(a1, a0, 0x0c060c02u) << 2) | 0x00010001u;
    const uint32_t k3 = __builtin_amdgcn_perm(a1, a0, 0x0c070c03u) << 2;
    const uint32_t m01 = max_u16x2(k0, k1);
    const uint32_t m3 = max_u16x2(m01, k2);
    const uint32_t med = max_u16x2(min_u16x2(k0, k1), min_u16x2(m01, k2));
    const uint32_t first = max_u16x2(m3, k3), second = max_u16x2(med, min_u16x2(m3, k3));
    const uint32_t pf = first & 0x00030003u, ps = second & 0x00030003u;  // 3 - position
    lo = max_u16x2(pf, ps) ^ 0x00030003u;
    hi = min_u16x2(pf, ps) ^ 0x00030003u;
}

// The int8 magnitude prune on the same grid as prune_compress_kernel: lane (r, qq) of wave w holds 32
// columns of row 16 b + r in tile t as two 16-byte words; each pair of groups yields 4 value bytes, gathered
// by one byte permute (selector 0-3: bytes of the even group's word, 4-7: of the odd one's), and 8 index bits.
template <int TPW>
__global__ __launch_bounds__(256) void prune_compress_i8_kernel(const void* __restrict__ W, int64_t ldw, int64_t M,
                                                                int64_t K, int64_t tiles, int64_t groups_x,
                                                                int8_t* __restrict__ values, uint8_t* __restrict__ meta) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, qq = lane >> 4;
    const int64_t b = blockIdx.x / groups_x;
    const int64_t tx = blockIdx.x - b * groups_x;
    const int64_t row = 16 * b + r;
    const bool row_ok = row < M;
    const char* wrow = reinterpret_cast<const char*>(W) + row * ldw;
    u32x4 x[TPW][2];
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int64_t t = tx * 4 * TPW + wave + 4 * i;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int64_t c = t * 128 + 32 * qq + 16 * h;  // K is a multiple of 16: a piece is all in or all out
            x[i][h] = u32x4{0, 0, 0, 0};
            if (row_ok && t < tiles && c < K) x[i][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + c));
        }
    }
#pragma unroll
    for (int i = 0; i < TPW; i++) {
        const int64_t t = tx * 4 * TPW + wave + 4 * i;
        if (t >= tiles) break;
        // zero words (past M or K) select positions 0 and 1 with zero values: the padding encoding
        uint32_t out[4], mbits = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t w0 = x[i][k >> 1][2 * (k & 1)], w1 = x[i][k >> 1][2 * (k & 1) + 1];
            uint32_t lo, hi;  // w0's positions in the low halves, w1's in the high halves
            top2_i8_pair(w0, w1, lo, hi);
            // selector lo0, hi0 (bytes of w0), lo1 + 4, hi1 + 4 (bytes of w1)
            out[k] = __builtin_amdgcn_perm(w1, w0, lo | (hi << 8) | 0x04040000u);
            // index bits lo0 | hi0 << 2 | lo1 << 4 | hi1 << 6
            const uint32_t e = lo | (hi << 2);
            mbits |= ((e | (e >> 12)) & 0xFFu) << (8 * k);
        }
        *reinterpret_cast<u32x4*>(values + (b * tiles + t) * 1024 + 16 * lane) = u32x4{out[0], out[1], out[2], out[3]};
        *reinterpret_cast<uint32_t*>(meta + (b * tiles + t) * 256 + 4 * lane) = mbits;
    }
}

// One thread per 16-column chunk of the M x K weight, numbered in the order of the compressed tiles: the 16
// rows of a row block first, then the chunk's place in the tile's 64-byte rows, then the tile. The lanes
// of a wave then read whole 1 KB value tiles and their metadata in address order, and (bf16) write 16
// full 128-byte row segments; numbered row by row, neighbouring lanes read 16 bytes 256 bytes apart
// (28672 x 8192 bf16: 223 us, 40 % of HBM).
template <int DT>
__global__ __launch_bounds__(256) void decompress_kernel(const void* __restrict__ values,
                                                         const uint8_t* __restrict__ meta, uint32_t M,
                                                         uint32_t chunks_per_row, uint32_t total_threads,
                                                         int64_t tiles_per_row, void* __restrict__ W, int64_t ldw) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= total_threads) return;
    constexpr int isz = esize<DT>();
    constexpr uint32_t CPT = 8 / isz;  // 16-column chunks per 64-byte tile row
    const uint32_t rest = t >> 4, cq = rest % CPT, tl = rest / CPT;
    const uint32_t blk = tl / (uint32_t)tiles_per_row, tt = tl - blk * (uint32_t)tiles_per_row;
    const uint32_t row = 16 * blk + (t & 15), c = tt * CPT + cq;
    if (row >= M || c >= chunks_per_row) return;
    constexpr int TM = 16 / isz;
    const char* vbase = reinterpret_cast<const char*>(values);
    const int64_t vb = 8 * isz * (int64_t)c;
    uint32_t mbits;
    if (TM >= 8) {
        mbits = *reinterpret_cast<const uint16_t*>(meta + tiled_offset<TM>(row, 2 * (int64_t)c, tiles_per_row));
    } else {
        mbits = meta[tiled_offset<TM>(row, 2 * (int64_t)c, tiles_per_row)] |
                ((uint32_t)meta[tiled_offset<TM>(row, 2 * (int64_t)c + 1, tiles_per_row)] << 8);
    }
    uint32_t v[8];
    if (isz == 2) {
        uint4 a = *reinterpret_cast<const uint4*>(vbase + tiled_offset<64>(row, vb, tiles_per_row));
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    } else if (isz == 4) {
        uint4 a = *reinterpret_cast<const uint4*>(vbase + tiled_offset<64>(row, vb, tiles_per_row));
        uint4 b = *reinterpret_cast<const uint4*>(vbase + tiled_offset<64>(row, vb + 16, tiles_per_row));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint2 a = *reinterpret_cast<const uint2*>(vbase + tiled_offset<64>(row, vb, tiles_per_row));
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = ((i < 4 ? a.x : a.y) >> (8 * (i & 3))) & 0xFFu;
    }
    uint32_t out[16];
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const uint32_t nib = (mbits >> (4 * g)) & 0xF;
        const uint32_t p0 = nib & 3, p1 = nib >> 2;
#pragma unroll
        for (int i = 0; i < 4; i++) out[4 * g + i] = (i == p0) ? v[2 * g] : ((i == p1) ? v[2 * g + 1] : 0u);
    }
    char* wp = reinterpret_cast<char*>(W) + ((int64_t)row * ldw + 16 * (int64_t)c) * isz;
    if (isz == 2) {
        uint4* o = reinterpret_cast<uint4*>(wp);
        o[0] = make_uint4(out[0] | (out[1] << 16), out[2] | (out[3] << 16), out[4] | (out[5] << 16),
                          out[6] | (out[7] << 16));
        o[1] = make_uint4(out[8] | (out[9] << 16), out[10] | (out[11] << 16), out[12] | (out[13] << 16),
                          out[14] | (out[15] << 16));
    } else if (isz == 4) {
        uint4* o = reinterpret_cast<uint4*>(wp);
#pragma unroll
        for (int i = 0; i < 4; i++) o[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            w[i] = out[4 * i] | (out[4 * i + 1] << 8) | (out[4 * i + 2] << 16) | (out[4 * i + 3] << 24);
        *reinterpret_cast<uint4*>(wp) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// k-of-4 masks (NVIDIA blog, progressive sparse training, Figure 4: keep 3 of every 4, later 2 of 4).
// One thread per 16-column chunk of a row: 4 groups; element t of a group is kept when fewer than
// `keep` others beat it (the selection rule above: larger key, or equal key and lower index). Writes
// the 4 mask nibbles (bit t = position t kept; 2 bytes of the row's K/8) and, when W_out is set, the
// masked chunk (kept elements bit-copied, +0 elsewhere).
template <int DT, bool WANDA>
__global__ __launch_bounds__(256) void prune_mask_kernel(const void* __restrict__ W, int64_t ldw, uint32_t chunks_per_row,
                                                         uint32_t total_chunks, int keep, const float* __restrict__ norms,
                                                         uint8_t* __restrict__ mask, int64_t mask_ld, void* __restrict__ W_out,
                                                         int64_t ldo) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= total_chunks) return;
    const uint32_t row = t / chunks_per_row, c = t - row * chunks_per_row;
    constexpr int isz = esize<DT>();
    typedef typename Elem<DT>::T T;
    const char* src = reinterpret_cast<const char*>(W) + ((int64_t)row * ldw + 16 * (int64_t)c) * isz;
    uint32_t w[4 * isz];  // the chunk's 16 elements as 4 * isz words
#pragma unroll
    for (int h = 0; h < isz; h++) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + h);
#pragma unroll
        for (int e = 0; e < 4; e++) w[4 * h + e] = v[e];
    }
    T x[16];
#pragma unroll
    for (int e = 0; e < 16; e++) {
        if (isz == 4) x[e] = (T)w[e];
        if (isz == 2) x[e] = (T)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        if (isz == 1) x[e] = (T)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
    }
    uint32_t bits = 0;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        uint32_t key[4];
#pragma unroll
        for (int e = 0; e < 4; e++) key[e] = select_key<DT, WANDA>(x[4 * g + e], WANDA ? norms[16 * c + 4 * g + e] : 0.f);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            int beaten_by = 0;
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (u != e) beaten_by += (key[u] > key[e] || (key[u] == key[e] && u < e)) ? 1 : 0;
            if (beaten_by < keep) bits |= 1u << (4 * g + e);
        }
    }
    if (mask) *reinterpret_cast<uint16_t*>(mask + (int64_t)row * mask_ld + 2 * (int64_t)c) = (uint16_t)bits;
    if (W_out) {
        uint32_t o[4 * isz];
#pragma unroll
        for (int k = 0; k < 4 * isz; k++) o[k] = 0;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const uint32_t v = (bits >> e) & 1 ? (uint32_t)x[e] : 0u;
            if (isz == 4) o[e] = v;
            if (isz == 2) o[e >> 1] |= v << (16 * (e & 1));
            if (isz == 1) o[e >> 2] |= v << (8 * (e & 3));
        }
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(W_out) + ((int64_t)row * ldo + 16 * (int64_t)c) * isz);
#pragma unroll
        for (int h = 0; h < isz; h++) dst[h] = make_uint4(o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]);
    }
}

template <int DT, bool WANDA>
static hipError_t launch_mask(const void* W, int64_t M, int64_t K, int64_t ldw, int keep, const float* norms,
                              uint8_t* mask, void* W_out, int64_t ldo, hipStream_t s) {
    const uint32_t cpr = (uint32_t)(K / 16);
    const uint32_t total = (uint32_t)(M * (K / 16));
    const uint32_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((prune_mask_kernel<DT, WANDA>), dim3(blocks), dim3(256), 0, s, W, ldw, cpr, total, keep, norms,
                       mask, K / 8, W_out, ldo);
    return hipGetLastError();
}

hipError_t launch_prune_mask(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int keep, int score,
                             const float* norms, uint8_t* mask, void* W_out, int64_t ldo, hipStream_t s) {
    const bool wanda = score == 1;
    switch (dtype) {
    case DT_BF16:
        return wanda ? launch_mask<DT_BF16, true>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s)
                     : launch_mask<DT_BF16, false>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s);
    case DT_FP16:
        return wanda ? launch_mask<DT_FP16, true>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s)
                     : launch_mask<DT_FP16, false>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s);
    case DT_FP32:
        return wanda ? launch_mask<DT_FP32, true>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s)
                     : launch_mask<DT_FP32, false>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s);
    case DT_I8:
        return launch_mask<DT_I8, false>(W, M, K, ldw, keep, norms, mask, W_out, ldo, s);
    }
    return hipErrorInvalidValue;
}

// Padded sizes of the compressed form (values of `vsz` bytes): Mp, Kp, tiles per row.
static inline void padded_dims(int64_t M, int64_t K, int vsz, int64_t& Mp, int64_t& Kp, int64_t& tiles) {
    const int64_t kt = 128 / vsz;
    Mp = (M + 15) / 16 * 16;
    Kp = (K + kt - 1) / kt * kt;
    tiles = Kp / kt;
}

template <int DT, int VOUT, bool WANDA, int TPW>
static hipError_t launch_pc_tpw(const void* W, int64_t M, int64_t K, int64_t ldw, const float* norms, void* values,
                                uint8_t* meta, int64_t Mp, int64_t tiles, hipStream_t s) {
    const int64_t groups_x = (tiles + 4 * TPW - 1) / (4 * TPW);
    const int64_t blocks = (Mp / 16) * groups_x;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if constexpr (DT == DT_I8)
        hipLaunchKernelGGL((prune_compress_i8_kernel<TPW>), dim3((unsigned)blocks), dim3(256), 0, s, W, ldw, M, K, tiles,
                           groups_x, static_cast<int8_t*>(values), meta);
    else
        hipLaunchKernelGGL((prune_compress_kernel<DT, VOUT, WANDA, TPW>), dim3((unsigned)blocks), dim3(256), 0, s, W,
                           ldw, M, K, tiles, groups_x, norms, values, meta);
    return hipGetLastError();
}

// One tile per wave: measured on MI355X against 2, 4 and 8 tiles per wave (more loads in flight per lane,
// fewer workgroups), one was the fastest at every size (28672 x 8192 bf16: 127.6 us against 142.8 us with
// four, 72 % of HBM; 11008 x 4096: 27.1 against 30.0 us; Wanda 146 against 150 us), the hardware keeping
// more, smaller workgroups in flight. The int8 kernel likewise (28672 x 8192: 86.6-89.0 us against 87.0-87.4
// with two).
template <int DT, int VOUT, bool WANDA>
static hipError_t launch_pc(const void* W, int64_t M, int64_t K, int64_t ldw, const float* norms, void* values,
                            uint8_t* meta, hipStream_t s) {
    int64_t Mp, Kp, tiles;
    padded_dims(M, K, esize<VOUT>(), Mp, Kp, tiles);
    return launch_pc_tpw<DT, VOUT, WANDA, 1>(W, M, K, ldw, norms, values, meta, Mp, tiles, s);
}

hipError_t launch_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                                 const float* norms, void* values, int val_dtype, uint8_t* meta, hipStream_t s) {
    const bool wanda = score == 1;
    switch (dtype) {
    case DT_BF16:
        return wanda ? launch_pc<DT_BF16, DT_BF16, true>(W, M, K, ldw, norms, values, meta, s)
                     : launch_pc<DT_BF16, DT_BF16, false>(W, M, K, ldw, norms, values, meta, s);
    case DT_FP16:
        return wanda ? launch_pc<DT_FP16, DT_FP16, true>(W, M, K, ldw, norms, values, meta, s)
                     : launch_pc<DT_FP16, DT_FP16, false>(W, M, K, ldw, norms, values, meta, s);
    case DT_FP32:
        if (val_dtype == DT_BF16)
            return wanda ? launch_pc<DT_FP32, DT_BF16, true>(W, M, K, ldw, norms, values, meta, s)
                         : launch_pc<DT_FP32, DT_BF16, false>(W, M, K, ldw, norms, values, meta, s);
        return wanda ? launch_pc<DT_FP32, DT_FP32, true>(W, M, K, ldw, norms, values, meta, s)
                     : launch_pc<DT_FP32, DT_FP32, false>(W, M, K, ldw, norms, values, meta, s);
    case DT_I8:
        return launch_pc<DT_I8, DT_I8, false>(W, M, K, ldw, norms, values, meta, s);
    }
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_dc(const void* values, const uint8_t* meta, int64_t M, int64_t K, void* W_out, int64_t ldw,
                            hipStream_t s) {
    int64_t Mp, Kp, tiles;
    padded_dims(M, K, esize<DT>(), Mp, Kp, tiles);
    const uint32_t cpr = (uint32_t)(K / 16);
    const uint32_t total = (uint32_t)(Mp * tiles * (8 / esize<DT>()));  // one thread per chunk of the padded tiles
    const uint32_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(decompress_kernel<DT>, dim3(blocks), dim3(256), 0, s, values, meta, (uint32_t)M, cpr, total,
                       tiles, W_out, ldw);
    return hipGetLastError();
}

hipError_t launch_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K, void* W_out,
                             int64_t ldw, hipStream_t s) {
    switch (dtype) {
    case DT_BF16:
    case DT_FP16: return launch_dc<DT_BF16>(values, meta, M, K, W_out, ldw, s);
    case DT_FP32: return launch_dc<DT_FP32>(values, meta, M, K, W_out, ldw, s);
    case DT_I8: return launch_dc<DT_I8>(values, meta, M, K, W_out, ldw, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sp24
