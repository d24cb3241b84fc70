// 2:4 prune + compress, and decompress (Orin NN design, Chapter 7, section 2.1 Steps 1-2; NVIDIA
// blog on Ampere structured sparsity, Figure 1).
//
// Both kernels are HBM streams. One thread owns one 16-column chunk of a row (4 groups): it reads
// the chunk with 16-byte loads, scores and selects in registers, and writes 8 values (one 16-byte
// store for 16-bit types) plus the chunk's 16 metadata bits (2 bytes) into the tiled compressed
// layout (16-row tiles in the order of the sparse MFMA operand). Consecutive threads own consecutive
// chunks of a row, so loads are contiguous runs; each store lands in a 16-byte quarter of a tile.
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

// Element storage for one 16-column chunk.
template <int DT> struct Chunk;
template <> struct Chunk<DT_BF16> {
    typedef uint16_t T;
    T e[16];
    __device__ void load(const void* p) {
        const u32x4* q = reinterpret_cast<const u32x4*>(p);
        u32x4 a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 1);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) { e[2 * i] = (T)(w[i] & 0xFFFF); e[2 * i + 1] = (T)(w[i] >> 16); }
    }
    __device__ uint32_t mag_key(int i) const { return e[i] & 0x7FFFu; }
    __device__ float abs_f32(int i) const { return bf16_to_f32(e[i] & 0x7FFFu); }
};
template <> struct Chunk<DT_FP16> : Chunk<DT_BF16> {
    __device__ float abs_f32(int i) const { return f16_to_f32(e[i] & 0x7FFFu); }
};
template <> struct Chunk<DT_FP32> {
    typedef uint32_t T;
    T e[16];
    __device__ void load(const void* p) {
        const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            u32x4 a = __builtin_nontemporal_load(q + i);
            e[4 * i] = a.x; e[4 * i + 1] = a.y; e[4 * i + 2] = a.z; e[4 * i + 3] = a.w;
        }
    }
    __device__ uint32_t mag_key(int i) const { return e[i] & 0x7FFFFFFFu; }
    __device__ float abs_f32(int i) const { return __uint_as_float(e[i] & 0x7FFFFFFFu); }
};
template <> struct Chunk<DT_I8> {
    typedef uint8_t T;
    T e[16];
    __device__ void load(const void* p) {
        u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 16; i++) e[i] = (T)((w[i >> 2] >> (8 * (i & 3))) & 0xFF);
    }
    __device__ uint32_t mag_key(int i) const {
        int v = (int)(int8_t)e[i];
        return (uint32_t)(v < 0 ? -v : v);
    }
    __device__ float abs_f32(int) const { return 0.f; }  // Wanda is not offered for int8
};

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

// One thread per 16-column chunk c of padded row i (Mp x Kp/16 chunks, Kp/KT tiles per row). Chunks
// outside the M x K weight write the padding (values 0, metadata nibbles 0x4).
template <int DT, int VOUT, bool WANDA>
__global__ __launch_bounds__(256) void prune_compress_kernel(const void* __restrict__ W, int64_t ldw, int64_t M,
                                                             int64_t K, uint32_t chunks_per_row, uint32_t total_chunks,
                                                             int64_t tiles_per_row, const float* __restrict__ norms,
                                                             void* __restrict__ values, uint8_t* __restrict__ meta) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= total_chunks) return;
    const uint32_t row = t / chunks_per_row, c = t - row * chunks_per_row;
    constexpr int isz = esize<DT>(), vsz = esize<VOUT>();
    typename Chunk<DT>::T kept[8];
    uint32_t mbits = 0x4444u;
    if (row < M && 16 * (int64_t)c < K) {
        Chunk<DT> x;
        x.load(reinterpret_cast<const char*>(W) + ((int64_t)row * ldw + 16 * (int64_t)c) * isz);
        float nrm[16];
        if (WANDA) {
            const float4* np = reinterpret_cast<const float4*>(norms + 16 * (int64_t)c);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float4 v = np[i];
                nrm[4 * i] = v.x; nrm[4 * i + 1] = v.y; nrm[4 * i + 2] = v.z; nrm[4 * i + 3] = v.w;
            }
        }
        mbits = 0;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            uint32_t key[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (WANDA)
                    key[i] = __float_as_uint(__fmul_rn(x.abs_f32(4 * g + i), nrm[4 * g + i])) & 0x7FFFFFFFu;
                else
                    key[i] = x.mag_key(4 * g + i);
            }
            int lo, hi;
            knockout_top2(key, lo, hi);
            mbits |= (uint32_t)(lo | (hi << 2)) << (4 * g);
            kept[2 * g] = x.e[4 * g + lo];
            kept[2 * g + 1] = x.e[4 * g + hi];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) kept[i] = 0;
    }
    // values: 8 kept values = 8 * vsz bytes at byte 8 * vsz * c of the compressed row
    char* vbase = reinterpret_cast<char*>(values);
    const int64_t vb = 8 * vsz * (int64_t)c;
    if (VOUT == DT_FP32) {  // two whole 16-byte quarters
        *reinterpret_cast<uint4*>(vbase + tiled_offset<64>(row, vb, tiles_per_row)) =
            make_uint4(kept[0], kept[1], kept[2], kept[3]);
        *reinterpret_cast<uint4*>(vbase + tiled_offset<64>(row, vb + 16, tiles_per_row)) =
            make_uint4(kept[4], kept[5], kept[6], kept[7]);
    } else if (VOUT == DT_I8) {  // half of a quarter
        uint2 v;
        v.x = (uint32_t)kept[0] | ((uint32_t)kept[1] << 8) | ((uint32_t)kept[2] << 16) | ((uint32_t)kept[3] << 24);
        v.y = (uint32_t)kept[4] | ((uint32_t)kept[5] << 8) | ((uint32_t)kept[6] << 16) | ((uint32_t)kept[7] << 24);
        *reinterpret_cast<uint2*>(vbase + tiled_offset<64>(row, vb, tiles_per_row)) = v;
    } else {  // 16-bit values: one quarter; bf16/fp16 bit copies, or fp32 rounded to bf16
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (DT == DT_FP32)
                h[i] = f32_to_bf16_rne(__uint_as_float((uint32_t)kept[i]));
            else
                h[i] = (uint32_t)kept[i];
        }
        *reinterpret_cast<uint4*>(vbase + tiled_offset<64>(row, vb, tiles_per_row)) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
    // metadata: 2 bytes at byte 2c of the row's metadata; tiles of KT/8 = 16/vsz bytes per row
    constexpr int TM = 16 / vsz;
    if (TM >= 8) {  // bf16 (quarter 2 bytes) and int8 (quarter 4 bytes): one 16-bit store
        *reinterpret_cast<uint16_t*>(meta + tiled_offset<TM>(row, 2 * (int64_t)c, tiles_per_row)) = (uint16_t)mbits;
    } else {  // fp32: 1-byte quarters
        meta[tiled_offset<TM>(row, 2 * (int64_t)c, tiles_per_row)] = (uint8_t)(mbits & 0xFF);
        meta[tiled_offset<TM>(row, 2 * (int64_t)c + 1, tiles_per_row)] = (uint8_t)(mbits >> 8);
    }
}

// One thread per 16-column chunk of the M x K weight.
template <int DT>
__global__ __launch_bounds__(256) void decompress_kernel(const void* __restrict__ values,
                                                         const uint8_t* __restrict__ meta, uint32_t chunks_per_row,
                                                         uint32_t total_chunks, int64_t tiles_per_row,
                                                         void* __restrict__ W, int64_t ldw) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= total_chunks) return;
    const uint32_t row = t / chunks_per_row, c = t - row * chunks_per_row;
    constexpr int isz = esize<DT>();
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

// Padded sizes of the compressed form (values of `vsz` bytes): Mp, Kp, tiles per row.
static inline void padded_dims(int64_t M, int64_t K, int vsz, int64_t& Mp, int64_t& Kp, int64_t& tiles) {
    const int64_t kt = 128 / vsz;
    Mp = (M + 15) / 16 * 16;
    Kp = (K + kt - 1) / kt * kt;
    tiles = Kp / kt;
}

template <int DT, int VOUT, bool WANDA>
static hipError_t launch_pc(const void* W, int64_t M, int64_t K, int64_t ldw, const float* norms, void* values,
                            uint8_t* meta, hipStream_t s) {
    int64_t Mp, Kp, tiles;
    padded_dims(M, K, esize<VOUT>(), Mp, Kp, tiles);
    const uint32_t cpr = (uint32_t)(Kp / 16);
    const uint32_t total = (uint32_t)(Mp * (Kp / 16));
    const uint32_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((prune_compress_kernel<DT, VOUT, WANDA>), dim3(blocks), dim3(256), 0, s, W, ldw, M, K, cpr, total,
                       tiles, norms, values, meta);
    return hipGetLastError();
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
    const uint32_t total = (uint32_t)(M * (K / 16));
    const uint32_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(decompress_kernel<DT>, dim3(blocks), dim3(256), 0, s, values, meta, cpr, total, tiles, W_out, ldw);
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
